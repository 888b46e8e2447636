#!/usr/bin/env python3
"""Benchmark of the packed lookahead + verification round on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full round (pool lookup, row manifest, target forward over the
packed rows, LM head on the required rows, verification, K/V commit, pool
upsert, window advance) through the C ABI's la_step.  Default workload, the
largest configuration that fits one GPU: a CodeLlama-34B-shaped random-init
bf16 decoder (48 layers, d 8192, 64 query heads on 8 KV heads, MLP 22016,
vocab 32000), 2048-token prompt from the seeded order-2 Markov chain with
~30% copied spans, greedy lookahead with W=15, N=7, G=15, 256 new tokens,
batch 1.  Weights and prompt are resident in HBM before timing; prefill is
outside the timed region.  value = emitted tokens / wall time of the K timed
rounds (K = --steps; 0 times one complete generation).

Also on the same line:
  * roofline: the dominant kernel of the step (the batch-invariant GEMM that
    streams the weights): algorithmic bytes per launch over its average
    launch time from HIP events on the library's stream;
  * cpu_baseline: the CPU oracle on a bounded slice of the same workload;
  * lookahead_attn (+ _8192, _34b_gqa): the isolated lookahead-mask attention
    op, bf16, timed with HIP events over rotating input sets larger than the
    256 MB Infinity Cache;
  * extra_workloads: the 7B-shaped workloads (512-token prompt, W=7 N=5 G=7;
    8192-token prompt, W=15 N=5 G=15 greedy and temperature-0.7 sampled over
    five prompt/sampler seeds), each with the same round measurements; and
    4, 8 and 16 of the 512-token requests decoded together by la_batch_step
    under a 256-row budget (aggregate tokens/s against the same requests
    batched autoregressively); and the tiny fp32 decoder of config 1, whose
    n-grams recur, over five prompt seeds against autoregressive decoding.
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
HEADLINE = "codellama34b_w15n7g15"

WORKLOADS = {
    "codellama34b_w15n7g15": dict(model="codellama34b", W=15, N=7, G=15, prompt=2048, max_new=256, copyspan=True,
                                  desc=("CodeLlama-34B-shaped bf16 decoder (48 layers, GQA 64/8 heads), 2048-token "
                                        "Markov prompt with ~30% copied spans, greedy lookahead W=15 N=7 G=15, "
                                        "256 new tokens, batch 1")),
    "llama7b_w7n5g7": dict(model="llama7b", W=7, N=5, G=7, prompt=512, max_new=256, desc=(
        "Llama-2-7B-shaped bf16 decoder, 512-token Markov prompt, greedy lookahead W=7 N=5 G=7, 256 new tokens")),
    "llama7b_long_w15n5g15": dict(model="llama7b", W=15, N=5, G=15, prompt=8192, max_new=256, desc=(
        "Llama-2-7B-shaped bf16 decoder, 8192-token Markov prompt, lookahead W=15 N=5 G=15, 256 new tokens")),
    "tiny_w5n3g5": dict(model="tiny", W=5, N=3, G=5, prompt=32, max_new=64, desc=(
        "tiny fp32 decoder (2 layers, d 64), 32-token Markov prompt, greedy lookahead W=5 N=3 G=5, 64 new tokens")),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_prompt(wl, dims, seed=0):
    import synthetic
    if wl.get("copyspan"):
        prompt, copied = synthetic.copyspan_prompt(dims.vocab, wl["prompt"], seed)
        return prompt, copied
    return synthetic.markov_prompt(dims.vocab, wl["prompt"], seed), 0.0


def measure_batch(model, dims, wl, n_req, budget, warmup, steps=0):
    """n_req requests of one workload (prompt seeds 0..n_req-1) decoded together
    by la_batch_step under a row budget: aggregate emitted tokens / wall time of
    the timed steps (steps == 0: every step after the warmup until all requests
    finish), the rows planned per step, and the same requests decoded
    autoregressively in one batch (one row each) with the same kernels."""
    import torch
    import exact_lookahead_decoding_amd.la as la

    def make(ar):
        ss = [la.Session(model, make_prompt(wl, dims, seed)[0], W=wl["W"], N=wl["N"], G=wl["G"],
                         max_new=wl["max_new"], ar_only=ar) for seed in range(n_req)]
        return ss, la.Batch(model, max_rows=256)

    res = {}
    for ar in (False, True):
        sessions, batch = make(ar)
        for _ in range(warmup):
            batch.la_batch_step(sessions, row_budget=budget)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tokens = done = rows = paused = found = verified = 0
        while steps == 0 or done < steps:
            toks, info = batch.la_batch_step(sessions, row_budget=budget)
            if all(i.Q == 0 for i in info):
                break
            tokens += sum(len(t) for t in toks)
            rows += sum(i.Q for i in info)
            paused += sum(i.paused for i in info)
            found += sum(i.found for i in info)
            verified += sum(i.verified for i in info)
            done += 1
        torch.cuda.synchronize()
        secs = time.perf_counter() - t0
        r = {"value": tokens / secs, "tokens": tokens, "steps": done, "ms_per_step": secs * 1e3 / done,
             "tokens_per_step": tokens / done, "rows_per_step": rows / done}
        if not ar:
            r.update(paused_rounds=paused, candidates_found=found, candidates_verified=verified)
            res.update(r)
        else:
            res["ar_batch_tokens_per_s"] = r["value"]
            res["ar_batch_ms_per_step"] = r["ms_per_step"]
            res["speedup_vs_ar_batch"] = res["value"] / r["value"]
        log(f"  batch {n_req} ({'autoregressive' if ar else 'lookahead'}, budget {budget}): {tokens} tokens in "
            f"{done} steps, {r['ms_per_step']:.3f} ms/step, {r['value']:.1f} tokens/s, "
            f"{r['rows_per_step']:.1f} rows/step")
        del sessions, batch
        torch.cuda.empty_cache()
    return res


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


def measure_tiny(warmup):
    """Config 1 (the tiny fp32 decoder, whose Markov-prompt n-grams recur in
    its own greedy continuations): one complete generation per prompt seed
    0..4, lookahead and autoregressive with the same kernels, aggregated."""
    import exact_lookahead_decoding_amd.la as la
    import synthetic
    dt = synthetic.PRESETS["tiny"]
    mt = la.DeviceModel(dt, seed=0)
    tw = WORKLOADS["tiny_w5n3g5"]
    runs = []
    for seed in range(5):
        log(f"tiny_w5n3g5 (prompt seed {seed}):")
        runs.append(measure(mt, dt, tw, 0, warmup, seed=seed, with_profile=False))
    secs = sum(r["rounds"] * r["ms_per_round"] * 1e-3 for r in runs)
    tokens = sum(r["tokens"] for r in runs)
    ar_secs = sum(r["tokens"] / r["ar_tokens_per_s"] for r in runs)   # the same tokens, autoregressively
    hist = [sum(r["accepted_hist"][i] for r in runs) for i in range(len(runs[0]["accepted_hist"]))]
    res = {"desc": tw["desc"] + "; one complete generation per prompt seed (a warmup session runs first), "
                                "against the same generations decoded autoregressively",
           "seeds": list(range(5)), "value": tokens / secs, "tokens": tokens,
           "rounds": sum(r["rounds"] for r in runs), "tokens_per_round": tokens / sum(r["rounds"] for r in runs),
           "ms_per_round": secs * 1e3 / sum(r["rounds"] for r in runs),
           "ar_tokens_per_s": tokens / ar_secs, "speedup_vs_ar": ar_secs / secs, "accepted_hist": hist,
           "value_per_seed": [r["value"] for r in runs],
           "tokens_per_round_per_seed": [r["tokens_per_round"] for r in runs]}
    log(f"  tiny: {res['value']:.1f} tokens/s, {res['tokens_per_round']:.3f} tokens/round, "
        f"{res['speedup_vs_ar']:.2f}x autoregressive")
    return res


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
        while done < steps:
            out = sess.la_step()
            if not out:
                break
            tokens += len(out)
            done += 1
        torch.cuda.synchronize()
        elapsed += time.perf_counter() - t0
        if done < steps:
            sess = make_session()
    return tokens, elapsed, sess, done


def kernel_rates(pr):
    """Per-launch averages of the GEMM and attention launches from la_profile's HIP events."""
    g_ms, a_ms = pr["gemm_ms"], pr["attn_ms"]
    return {
        "gemm_launches": pr["gemm_launches"],
        "gemm_avg_launch_us": g_ms / max(1, pr["gemm_launches"]) * 1e3,
        "gemm_bytes_per_launch": pr["gemm_bytes"] / max(1, pr["gemm_launches"]),
        "gemm_GBps": pr["gemm_bytes"] / (g_ms * 1e-3) / 1e9 if g_ms > 0 else 0.0,
        "gemm_ms_total": g_ms,
        "attn_launches": pr["attn_launches"],
        "attn_avg_launch_us": a_ms / max(1, pr["attn_launches"]) * 1e3,
        "attn_GBps": pr["attn_bytes"] / (a_ms * 1e-3) / 1e9 if a_ms > 0 else 0.0,
        "attn_ms_total": a_ms,
    }


def measure(model, dims, wl, steps, warmup, verify="greedy", temperature=0.7, seed=0, with_ar=True,
            with_profile=True, pool_from_prompt=False):
    """Lookahead rounds of one workload (prompt and sampler seed `seed`): tokens/s,
    rounds, the same generation autoregressively with the same kernels, and a
    separate HIP-event pass over the GEMM and attention launches."""
    import torch
    import exact_lookahead_decoding_amd.la as la
    prompt, copied = make_prompt(wl, dims, seed)
    vm = la.LA_VERIFY_SAMPLE if verify == "sample" else la.LA_VERIFY_GREEDY

    def make(ar=False, profile=False):
        s = la.Session(model, prompt, W=wl["W"], N=wl["N"], G=wl["G"], max_new=wl["max_new"], ar_only=ar,
                       verify_mode=vm, temperature=temperature, seed=seed,
                       pool_from_prompt=pool_from_prompt and not ar)
        if profile:
            s.la_profile(True)
        return s

    torch.cuda.synchronize()
    t = time.perf_counter()
    sess = make()
    torch.cuda.synchronize()
    init_prefill_ms = (time.perf_counter() - t) * 1e3
    for _ in range(warmup):
        sess.la_step()
    tokens, secs, sess, done = run_steps(make, sess, steps)
    st = sess.la_stats()
    res = {"value": tokens / secs, "tokens": tokens, "rounds": done, "ms_per_round": secs * 1e3 / done,
           "tokens_per_round": tokens / done, "init_prefill_ms": init_prefill_ms,
           "step_roofline": step_roofline(model, dims, wl, tokens, done, secs),
           "accepted_hist": st["hist"][: wl["N"] + 2], "copied_fraction": copied}
    log(f"  lookahead: {tokens} tokens in {done} rounds, {res['ms_per_round']:.3f} ms/round, "
        f"{res['value']:.1f} tokens/s, {res['tokens_per_round']:.3f} tokens/round")
    if with_ar:
        ar = make(ar=True)
        for _ in range(warmup):
            ar.la_step()
        ar_tokens, ar_secs, _, ar_done = run_steps(lambda: make(ar=True), ar, steps)
        res["ar_tokens_per_s"] = ar_tokens / ar_secs
        res["ar_ms_per_step"] = ar_secs * 1e3 / ar_done
        res["speedup_vs_ar"] = res["value"] / res["ar_tokens_per_s"]
        log(f"  autoregressive: {ar_tokens} tokens in {ar_done} steps, {res['ar_tokens_per_s']:.1f} tokens/s")
    if with_profile:
        prof = make(profile=True)
        for _ in range(warmup):
            prof.la_step()
        prof.la_profile(True)
        _, psecs, pend, pdone = run_steps(lambda: make(profile=True), prof, steps)
        rates = kernel_rates((pend if steps == 0 else prof).la_profile_read())
        rates["share_of_round_gemm"] = rates["gemm_ms_total"] / (psecs * 1e3)
        rates["share_of_round_attn"] = rates["attn_ms_total"] / (psecs * 1e3)
        res["kernels"] = rates
        log(f"  gemm: {rates['gemm_launches']} launches, avg {rates['gemm_avg_launch_us']:.1f} us, "
            f"{rates['gemm_GBps']:.0f} GB/s, {rates['share_of_round_gemm'] * 100:.0f}% of the rounds; attention: "
            f"avg {rates['attn_avg_launch_us']:.1f} us, {rates['attn_GBps']:.0f} GB/s")
    return res


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
    mk = lambda *s: torch.randn(*s, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)  # noqa
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
    flops = 4.0 * Q * H * dh * (p + 1 + info.maxp)
    gbs = alg / (ms * 1e-3) / 1e9
    kv_gbs = (2 * Hkv * p * dh * 2) / (ms * 1e-3) / 1e9
    heads = f"{H} heads" if H == Hkv else f"{H} query heads on {Hkv} KV heads"
    return {"workload": f"lookahead-mask attention, bf16, {heads} x 128, prefix {p}, {Q} rows (W=15 N={N} G=15)",
            "avg_us": ms * 1e3, "algorithmic_bytes": alg, "achieved_GBps": gbs, "kv_stream_GBps": kv_gbs,
            "peak_GBps": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS, "mfma_TFLOPs": flops / (ms * 1e-3) / 1e12,
            "reps": reps, "input_sets": sets}


ATTN_OPS = [dict(), dict(reps=24, sets=4, p=8192), dict(reps=64, sets=32, p=2048, H=64, Hkv=8, N=7)]
ATTN_KEYS = ["lookahead_attn", "lookahead_attn_8192", "lookahead_attn_34b_gqa"]

TRAFFIC_MD = os.path.join(ROOT, "profiles", "{kernel}_{wl}_hbm_traffic.md")
GEMM_SRC = os.path.join(ROOT, "exact_lookahead_decoding_amd", "csrc", "la_gemm.hip")
COPY_BYTES = 1 << 30


def gemm_kernel(wl_name):
    """The GEMM kernel a workload's rounds run: la_gemm2_kernel (bf16, 32x32x16 MFMA) or la_gemm_kernel (fp32)."""
    import synthetic
    return "la_gemm2_kernel" if synthetic.PRESETS[WORKLOADS[wl_name]["model"]].dtype == "bf16" else "la_gemm_kernel"


def _is_gemm(k):
    return "la_gemm_kernel" in k or "la_gemm2_kernel" in k


def _sha256(path):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def gemm_traffic(wl_name):
    """HBM bytes per round GEMM launch from the committed counter summary of the
    workload, or None when the GEMM source changed since the counters were taken."""
    try:
        txt = open(TRAFFIC_MD.format(kernel=gemm_kernel(wl_name), wl=wl_name)).read()
    except OSError:
        return None
    vals = dict(l.split(":", 1) for l in txt.splitlines() if l.startswith(("traffic_bytes_per_launch:",
                                                                               "la_gemm.hip sha256:")))
    if vals.get("la_gemm.hip sha256", "").strip() != _sha256(GEMM_SRC):
        return None
    return float(vals["traffic_bytes_per_launch"])


def profile_rounds(wl_name, rounds, warmup=5, verify="greedy"):
    """The workload's lookahead rounds alone (after prefill and warmup rounds),
    with HIP events around every GEMM and attention launch, then a plain copy
    of COPY_BYTES that calibrates the FETCH_SIZE / WRITE_SIZE counters.  The
    rounds' launches are the last GEMM / attention dispatches of the process
    before the copy; the JSON line says how many there were."""
    import torch
    import synthetic
    import exact_lookahead_decoding_amd.la as la
    la.load()
    torch.cuda.set_device(0)
    wl = WORKLOADS[wl_name]
    dims = synthetic.PRESETS[wl["model"]]
    model = la.DeviceModel(dims, seed=0)
    prompt, _ = make_prompt(wl, dims, 0)
    vm = la.LA_VERIFY_SAMPLE if verify == "sample" else la.LA_VERIFY_GREEDY
    sess = la.Session(model, prompt, W=wl["W"], N=wl["N"], G=wl["G"], max_new=wl["max_new"], verify_mode=vm,
                      temperature=0.7, seed=0)
    for _ in range(warmup):
        sess.la_step()
    torch.cuda.synchronize()
    sess.la_profile(True)
    t = time.perf_counter()
    for _ in range(rounds):
        sess.la_step()
    torch.cuda.synchronize()
    secs = time.perf_counter() - t
    pr = sess.la_profile_read()
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"workload": wl_name, "verify": verify, "rounds": rounds, "ms_per_round": secs * 1e3 / rounds,
                      "copy_bytes": COPY_BYTES, **kernel_rates(pr)}), flush=True)


def _dispatches(db_or_csv):
    """(kernel name, duration ns, counter values) per dispatch, in dispatch order,
    from a rocprofv3 results database or kernel-trace CSV."""
    if db_or_csv.endswith(".csv"):
        import csv
        rows = []
        with open(db_or_csv) as f:
            for r in csv.DictReader(f):
                rows.append((int(r.get("Dispatch_Id", len(rows))), r["Kernel_Name"],
                             int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        rows.sort()
        return [(k, d, {}) for _, k, d in rows]
    import sqlite3
    con = sqlite3.connect(db_or_csv)
    out = {}
    for d, k, c, v in con.execute("select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        e = out.setdefault(d, [k, 0, {}])
        e[2][c] = e[2].get(c, 0.0) + v
    return [tuple(out[d]) for d in sorted(out)]


def _round_gemms(disp, n):
    """The last n GEMM dispatches before the calibration copy."""
    gemm = [i for i, (k, _, _) in enumerate(disp) if _is_gemm(k) or "la_gemm_reduce_kernel" in k]
    return [disp[i] for i in gemm[-n:]]


def trace_summary(trace_csv, run_json, out_md, cmd):
    """Average duration of the rounds' GEMM and attention launches from a
    rocprofv3 kernel trace, next to the HIP-event averages of the same run."""
    import collections
    run = json.loads(open(run_json).read().strip().splitlines()[-1])
    disp = _dispatches(trace_csv)
    # a GEMM launch with split K is the GEMM kernel plus its reduction kernel (or, for the
    # residual projections, nothing: the next RMSNorm folds the partials)
    names = [k for k, _, _ in disp]
    g_idx = [i for i, k in enumerate(names) if _is_gemm(k) or "la_gemm_reduce_kernel" in k]
    a_idx = [i for i, k in enumerate(names) if "la_attn_kernel" in k or "la_attn_merge_kernel" in k]
    last_copy = max([i for i, k in enumerate(names) if "copy" in k.lower()] or [len(names)])
    g_idx = [i for i in g_idx if i < last_copy]
    a_idx = [i for i in a_idx if i < last_copy]
    # HIP-event brackets cover a GEMM kernel and its reduction together
    g_main = [i for i in g_idx if _is_gemm(names[i])][-run["gemm_launches"]:]
    first = g_main[0]
    g_sel = [i for i in g_idx if i >= first]
    a_main = [i for i in a_idx if "la_attn_kernel" in names[i]][-run["attn_launches"]:]
    a_sel = [i for i in a_idx if i >= a_main[0]] if a_main else []
    g_us = sum(disp[i][1] for i in g_sel) / 1e3 / len(g_main)
    a_us = sum(disp[i][1] for i in a_sel) / 1e3 / max(1, len(a_main))
    per = collections.defaultdict(lambda: [0, 0.0])
    for i in g_sel + a_sel:
        per[names[i]][0] += 1
        per[names[i]][1] += disp[i][1] / 1e3
    sampled = ", sampled verification (temperature 0.7)" if run.get("verify") == "sample" else ""
    lines = [f"# Kernel trace of the rounds: {run['workload']} ({WORKLOADS[run['workload']]['desc']}{sampled})", "",
             "Command (run from /tmp with TMPDIR=/tmp on one MI355X):", "", "```", cmd, "```", "",
             f"{run['rounds']} lookahead rounds after prefill and 5 warmup rounds, "
             f"{run['ms_per_round']:.3f} ms per round in the traced run.", "",
             "| kernel | calls | total us | avg us |", "|---|---:|---:|---:|"]
    for k, (c, t) in sorted(per.items(), key=lambda x: -x[1][1]):
        lines.append(f"| `{k[:90]}` | {c} | {t:.0f} | {t / c:.2f} |")
    # every kernel of the timed rounds: the dispatches from the first round GEMM up to the copy
    span = collections.defaultdict(lambda: [0, 0.0])
    for i in range(first, last_copy):
        span[names[i]][0] += 1
        span[names[i]][1] += disp[i][1] / 1e3
    busy = sum(t for _, t in span.values())
    lines += ["", f"All kernels of the {run['rounds']} rounds (per round; GPU busy {busy / run['rounds'] / 1e3:.3f} ms "
              f"of {run['ms_per_round']:.3f} ms):", "",
              "| kernel | calls per round | us per round | share of busy |", "|---|---:|---:|---:|"]
    for k, (c, t) in sorted(span.items(), key=lambda x: -x[1][1]):
        lines.append(f"| `{k[:90]}` | {c / run['rounds']:.1f} | {t / run['rounds']:.1f} | {t / busy * 100:.1f}% |")
    lines += ["", "| quantity | rocprofv3 trace | HIP events (same run) |", "|---|---:|---:|",
              f"| GEMM launches | {len(g_main)} | {run['gemm_launches']} |",
              f"| GEMM average launch (us) | {g_us:.2f} | {run['gemm_avg_launch_us']:.2f} |",
              f"| GEMM algorithmic bytes per launch (MB) | | {run['gemm_bytes_per_launch'] / 1e6:.2f} |",
              f"| GEMM GB/s | {run['gemm_bytes_per_launch'] / (g_us * 1e-6) / 1e9:.0f} | {run['gemm_GBps']:.0f} |",
              f"| attention launches | {len(a_main)} | {run['attn_launches']} |",
              f"| attention average launch, with split merge (us) | {a_us:.2f} | {run['attn_avg_launch_us']:.2f} |",
              "", "A GEMM launch is the GEMM kernel plus, where K is split and the output is not a residual,",
              "its reduction kernel; an attention launch is the attention kernel plus its split merge.", ""]
    md = "\n".join(lines)
    open(out_md, "w").write(md)
    print(md)


def pmc_summary(fetch_db, write_db, run_json, wl_name):
    """Per-launch HBM traffic of the rounds' GEMMs from a FETCH_SIZE and a
    WRITE_SIZE run of --profile-rounds, each scaled by what the counter reads
    for the calibration copy."""
    run = json.loads(open(run_json).read().strip().splitlines()[-1])
    out = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        disp = _dispatches(db)
        names = [k for k, _, _ in disp]
        # the calibration copies are the process's last three copy dispatches
        copies = [i for i, k in enumerate(names) if "copy" in k.lower()][-3:]
        end = copies[0] if copies else len(names)
        g = [i for i in range(end) if _is_gemm(names[i]) or "la_gemm_reduce_kernel" in names[i]]
        main = [i for i in g if _is_gemm(names[i])][-run["gemm_launches"]:]
        sel = [i for i in g if i >= main[0]]
        tot = sum(disp[i][2].get(counter, 0.0) for i in sel)
        copy = max(disp[i][2].get(counter, 0.0) for i in copies) if copies else 0.0
        out[counter] = (tot / len(main), copy, len(main))
    f_gemm, f_copy, n = out["FETCH_SIZE"]
    w_gemm, w_copy, _ = out["WRITE_SIZE"]
    ff = run["copy_bytes"] / (f_copy * 1024.0)
    fw = run["copy_bytes"] / (w_copy * 1024.0)
    fetch = f_gemm * 1024.0 * ff
    write = w_gemm * 1024.0 * fw
    alg = run["gemm_bytes_per_launch"]
    wl = WORKLOADS[wl_name]
    return "\n".join([
        f"# HBM traffic of the round GEMM: {wl_name} ({wl['desc']})",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp on one MI355X; each counter in a run of its own):",
        "",
        "```",
        f"python3 bench.py --profile-rounds {run['rounds']} --workload {wl_name} > out/run.json",
        f"rocprofv3 --pmc FETCH_SIZE -d out/pmc_fetch -o f -- python3 bench.py --profile-rounds {run['rounds']} "
        f"--workload {wl_name}",
        f"rocprofv3 --pmc WRITE_SIZE -d out/pmc_write -o w -- python3 bench.py --profile-rounds {run['rounds']} "
        f"--workload {wl_name}",
        f"python3 bench.py --pmc-summary out/pmc_fetch/f_results.db out/pmc_write/w_results.db out/run.json "
        f"--workload {wl_name}",
        "```",
        "",
        f"The run makes {run['rounds']} lookahead rounds after prefill and warmup, then copies a "
        f"{run['copy_bytes'] >> 20} MiB buffer three times.  Round GEMM launches: the last {n} `{gemm_kernel(wl_name)}` "
        "dispatches before the copy (with the split-K reductions that follow them).",
        "",
        "| quantity | value |",
        "|---|---:|",
        f"| copy: FETCH_SIZE (KiB) | {f_copy:.0f} |",
        f"| copy: WRITE_SIZE (KiB) | {w_copy:.0f} |",
        f"| FETCH_SIZE scale (copy bytes / counter bytes) | {ff:.3f} |",
        f"| WRITE_SIZE scale | {fw:.3f} |",
        f"| round GEMM launch: mean FETCH_SIZE (KiB) | {f_gemm:.0f} |",
        f"| round GEMM launch: mean WRITE_SIZE (KiB) | {w_gemm:.0f} |",
        f"| HBM read per launch, scaled (MB) | {fetch / 1e6:.2f} |",
        f"| HBM write per launch, scaled (MB) | {write / 1e6:.2f} |",
        f"| algorithmic bytes per launch (MB) | {alg / 1e6:.2f} |",
        f"| traffic / algorithmic | {(fetch + write) / alg:.3f} |",
        "",
        f"traffic_bytes_per_launch: {fetch + write:.0f}",
        f"la_gemm.hip sha256: {_sha256(GEMM_SRC)}",
        "",
    ])


def attn_summary(trace_csv, fetch_db, write_db, run_jsonl, out_md):
    """Kernel time and HBM traffic of the isolated attention op per shape, from a
    kernel trace and a FETCH_SIZE and a WRITE_SIZE run of
    `--attention-op-only --calibrate` (each launch: la_attn_kernel and, with
    several key splits, la_attn_merge_kernel); shapes are told apart by the
    attention kernel's grid, in the order the op runs them."""
    runs = [json.loads(l) for l in open(run_jsonl) if l.startswith("{")]

    def per_shape(disp, value):
        # consecutive attention dispatches of one grid size form a shape; a merge follows its kernel
        shapes, cur, grid = [], None, None
        for i, (k, dur, ctr, gsz) in enumerate(disp):
            if "la_attn_kernel" in k:
                if gsz != grid:
                    cur = {"grid": gsz, "attn": [], "merge": []}
                    shapes.append(cur)
                    grid = gsz
                cur["attn"].append(value(dur, ctr))
            elif "la_attn_merge_kernel" in k and cur is not None:
                cur["merge"].append(value(dur, ctr))
        return shapes

    import csv
    tr = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            tr.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                       {}, int(r["Grid_Size_X"]) if "Grid_Size_X" in r else int(r.get("Grid_Size", 0))))
    tr.sort()
    t_shapes = per_shape([x[1:] for x in tr], lambda d, c: d / 1e3)

    def pmc(db, counter):
        import sqlite3
        con = sqlite3.connect(db)
        rows = {}
        for d, k, c, v, gsz in con.execute("select dispatch_id, kernel_name, counter_name, value, grid_size "
                                           "from counters_collection"):
            e = rows.setdefault(d, [k, 0, {}, gsz])
            e[2][c] = e[2].get(c, 0.0) + v
        disp = [tuple(rows[d]) for d in sorted(rows)]
        copies = [i for i, x in enumerate(disp) if "copy" in x[0].lower()][-3:]
        cal = COPY_BYTES / (max(disp[i][2].get(counter, 0.0) for i in copies) * 1024.0)
        return per_shape(disp, lambda d, c: c.get(counter, 0.0) * 1024.0 * cal), cal

    f_shapes, f_cal = pmc(fetch_db, "FETCH_SIZE")
    w_shapes, w_cal = pmc(write_db, "WRITE_SIZE")
    mean = lambda v: sum(v) / len(v) if v else 0.0  # noqa: E731
    lines = ["# Lookahead-mask attention op: kernel time and HBM traffic per shape", "",
             "Commands (run from /tmp with TMPDIR=/tmp on one MI355X; each counter in a run of its own):", "", "```",
             "python3 bench.py --attention-op-only --calibrate > out/run.jsonl",
             "rocprofv3 --kernel-trace --stats --output-format csv -d out/trace -o a -- "
             "python3 bench.py --attention-op-only --calibrate",
             "rocprofv3 --pmc FETCH_SIZE -d out/pmc_fetch -o f -- python3 bench.py --attention-op-only --calibrate",
             "rocprofv3 --pmc WRITE_SIZE -d out/pmc_write -o w -- python3 bench.py --attention-op-only --calibrate",
             "python3 bench.py --attn-summary out/trace/a_kernel_trace.csv out/pmc_fetch/f_results.db "
             "out/pmc_write/w_results.db out/run.jsonl profiles/<this file>", "```", "",
             "Each shape runs eager warm-up launches, then HIP-graph replays of one launch per rotating input set "
             "(more bytes than the 256 MB Infinity Cache); the trace and counter averages below take every launch "
             "of the shape.  Counters are scaled by what they read for a plain 1 GiB copy "
             f"(FETCH_SIZE x{f_cal:.3f}, WRITE_SIZE x{w_cal:.3f}).", "",
             "| shape | launches | attention kernel avg us | merge avg us | kernel + merge us | HIP events us "
             "(op timing, graph) | algorithmic MB | HBM read MB | HBM write MB | traffic / algorithmic | "
             "achieved GB/s (events) | % of 8 TB/s |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for i, run in enumerate(runs):
        ts = t_shapes[i] if i < len(t_shapes) else {"attn": [], "merge": []}
        fs = f_shapes[i] if i < len(f_shapes) else {"attn": [], "merge": []}
        ws = w_shapes[i] if i < len(w_shapes) else {"attn": [], "merge": []}
        ka, km = mean(ts["attn"]), mean(ts["merge"])
        rd = mean(fs["attn"]) + mean(fs["merge"])
        wr = mean(ws["attn"]) + mean(ws["merge"])
        alg = run["algorithmic_bytes"]
        lines.append(f"| {run['workload']} | {len(ts['attn'])} | {ka:.2f} | {km:.2f} | {ka + km:.2f} | "
                     f"{run['avg_us']:.2f} | {alg / 1e6:.2f} | {rd / 1e6:.2f} | {wr / 1e6:.2f} | "
                     f"{(rd + wr) / alg:.2f} | {run['achieved_GBps']:.0f} | {run['frac'] * 100:.1f} |")
    lines += ["", "Algorithmic bytes: the committed K/V read once, each packed row's K/V, Q in and O out (bf16).  "
              "Traffic above it is the split states' round trip (fp32 partial O, m and l of every key split, "
              "written by the attention kernel and read by the merge) and re-reads.", ""]
    md = "\n".join(lines)
    open(out_md, "w").write(md)
    print(md)


def cpu_baseline(wl_name, rounds=1, prefix=32):
    """The oracle as it stands, on host cores, over a bounded slice of the workload:
    the same W/N/G and model widths, the first `prefix` tokens of the prompt
    (prefill untimed), the first steady rounds timed.  For the 34B shape a
    2-layer slice of the model (its first two layers, same seeded weights) runs
    and the round time is scaled by 48/2 (the LM head and round bookkeeping,
    counted 24 times, make the scaled time an overestimate)."""
    import dataclasses
    import numpy as np
    import synthetic
    from oracle.decode import lookahead_generate
    from oracle.model import OracleModel
    wl = WORKLOADS[wl_name]
    dims = synthetic.PRESETS[wl["model"]]
    layers = dims.n_layers
    if wl["model"] == "codellama34b":
        dims = dataclasses.replace(dims, n_layers=2)
    t = time.time()
    w = synthetic.model_weights(dims, 0)
    gen_s = time.time() - t
    prompt, _ = make_prompt(wl, dims, 0)
    prompt = prompt[:prefix]
    om = OracleModel(dims, w)
    times = []
    warm = wl["N"] - 2                      # warmup rounds before the window is complete
    res = lookahead_generate(om, prompt, wl["W"], wl["N"], wl["G"], 1 + warm + rounds, round_times=times)
    steady = times[warm:warm + rounds]
    toks = sum(len(r.emitted) for r in res["rounds"][warm:warm + rounds])
    scale = layers / dims.n_layers
    secs = sum(steady) * scale
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    q = [r.Q for r in res["rounds"][warm:warm + rounds]]
    slice_txt = (f"{dims.n_layers} of the {layers} layers (layers 0-1, same seeded weights), round time scaled by "
                 f"{scale:g}" if scale != 1 else "all layers")
    return {"value": toks / secs, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"numpy fp64 oracle, same model widths and W/N/G, {slice_txt}; prompt cut to its first "
                       f"{prefix} tokens, prefill and {warm} warmup rounds untimed, then {rounds} steady rounds "
                       f"({q} packed rows, {toks} tokens) in {sum(steady):.1f} s unscaled; weights generated in "
                       f"{gen_s:.0f} s outside the timing")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="rounds to time; 0 (default) times one complete generation of the workload")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attn", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the 7B-shaped extra workloads")
    ap.add_argument("--pool-from-prompt", action="store_true",
                    help="seed the n-gram pool with the prompt's n-grams (lookahead sessions)")
    ap.add_argument("--attention-op-only", action="store_true", help="time only the isolated attention op")
    ap.add_argument("--calibrate", action="store_true",
                    help="with --attention-op-only: end with three copies of COPY_BYTES (counter calibration)")
    ap.add_argument("--attn-summary", nargs=5, metavar=("TRACE_CSV", "FETCH_DB", "WRITE_DB", "RUN_JSONL", "OUT_MD"),
                    help="write the attention op's kernel-time and HBM-traffic summary under profiles/")
    ap.add_argument("--profile-rounds", type=int, default=0,
                    help="run only N rounds of --workload with kernel events (for rocprofv3 runs)")
    ap.add_argument("--verify", choices=("greedy", "sample"), default="greedy",
                    help="with --profile-rounds (and --trace-summary): the verification of the rounds "
                         "(sample: temperature 0.7, sampler seed 0)")
    ap.add_argument("--trace-summary", nargs=3, metavar=("TRACE_CSV", "RUN_JSON", "OUT_MD"))
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DB", "WRITE_DB", "RUN_JSON"),
                    help="write the GEMM traffic summary under profiles/ from two counter runs")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(*args.trace_summary, cmd=" ".join(
            ["rocprofv3 --kernel-trace --stats --output-format csv -d out/trace -o t -- python3 bench.py",
             f"--profile-rounds N --workload {args.workload}"]
            + ([f"--verify {args.verify}"] if args.verify != "greedy" else [])))
        return
    if args.pmc_summary:
        md = pmc_summary(*args.pmc_summary, args.workload)
        open(TRAFFIC_MD.format(kernel=gemm_kernel(args.workload), wl=args.workload), "w").write(md)
        print(md)
        return
    if args.profile_rounds:
        profile_rounds(args.workload, args.profile_rounds, verify=args.verify)
        return
    if args.attn_summary:
        attn_summary(*args.attn_summary)
        return
    if args.attention_op_only:
        import torch
        torch.cuda.set_device(0)
        for kw in ATTN_OPS:
            print(json.dumps(attention_op(**kw)), flush=True)
        if args.calibrate:
            src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
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
    log(f"{args.workload}: weights on device, {model.weight_bytes / 1e9:.2f} GB in {time.time() - t:.1f} s")
    head = measure(model, dims, wl, args.steps, args.warmup, pool_from_prompt=args.pool_from_prompt)
    k = head["kernels"]
    traffic = gemm_traffic(args.workload)
    line = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": head["rounds"],
        "warmup": args.warmup, "ms_per_step": head["ms_per_round"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if dims.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": wl["desc"], "W": wl["W"], "N": wl["N"], "G": wl["G"], "prompt_tokens": wl["prompt"],
                   "max_new": wl["max_new"], "verify": "greedy", "batch": 1,
                   "pool_from_prompt": bool(args.pool_from_prompt)},
        "roofline": {"bound": "hbm", "achieved": k["gemm_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": k["gemm_GBps"] / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": gemm_kernel(args.workload) + " (+ split reduction): every projection, MLP and "
                               "LM-head launch of the timed rounds",
                     "avg_launch_us": k["gemm_avg_launch_us"], "algorithmic_bytes_per_launch":
                         k["gemm_bytes_per_launch"], "launches": k["gemm_launches"],
                     "share_of_round": k["share_of_round_gemm"]},
    }
    for key in ("tokens_per_round", "ar_tokens_per_s", "ar_ms_per_step", "speedup_vs_ar", "step_roofline",
                "init_prefill_ms", "accepted_hist", "copied_fraction"):
        line[key] = head[key]
    line["attention_in_step"] = {"achieved_GBps": k["attn_GBps"], "avg_launch_us": k["attn_avg_launch_us"],
                                 "launches": k["attn_launches"], "share_of_round": k["share_of_round_attn"]}
    log(f"headline: {head['value']:.2f} tokens/s, GEMM {k['gemm_GBps']:.0f} GB/s "
        f"({k['gemm_GBps'] / HBM_PEAK_GBS * 100:.1f}% of HBM peak)")
    if not args.no_attn:
        for key, kw in zip(ATTN_KEYS, ATTN_OPS):
            a = attention_op(**kw)
            log(f"{key}: {a['avg_us']:.2f} us, {a['achieved_GBps']:.0f} GB/s ({a['frac'] * 100:.1f}%)")
            line[key] = a
    if not args.no_cpu_baseline:
        t = time.time()
        line["cpu_baseline"] = cpu_baseline(args.workload)
        log(f"cpu baseline: {line['cpu_baseline']['value']:.5f} tokens/s ({time.time() - t:.0f} s)")
    if not args.no_extras and args.workload == HEADLINE:
        del model
        torch.cuda.empty_cache()
        extras = {}
        d7 = synthetic.PRESETS["llama7b"]
        t = time.time()
        m7 = la.DeviceModel(d7, seed=0)
        log(f"7B-shaped weights on device in {time.time() - t:.1f} s")
        log("llama7b_w7n5g7 (greedy):")
        extras["llama7b_w7n5g7"] = dict(desc=WORKLOADS["llama7b_w7n5g7"]["desc"],
                                        **measure(m7, d7, WORKLOADS["llama7b_w7n5g7"], args.steps, args.warmup))
        long = WORKLOADS["llama7b_long_w15n5g15"]
        for mode in ("greedy", "sample"):
            runs = []
            for seed in range(5):
                log(f"llama7b_long_w15n5g15 ({mode}, seed {seed}):")
                runs.append(measure(m7, d7, long, args.steps, args.warmup, verify=mode, temperature=0.7, seed=seed,
                                    with_ar=seed == 0, with_profile=seed == 0))
            agg = {"desc": long["desc"] + (", temperature-0.7 one-hot sampling" if mode == "sample" else
                                           ", greedy"),
                   "seeds": list(range(5)), "value": sum(r["tokens"] for r in runs) / sum(
                       r["rounds"] * r["ms_per_round"] * 1e-3 for r in runs),
                   "value_per_seed": [r["value"] for r in runs],
                   "tokens_per_round": sum(r["tokens"] for r in runs) / sum(r["rounds"] for r in runs),
                   "ms_per_round": sum(r["rounds"] * r["ms_per_round"] for r in runs) / sum(r["rounds"]
                                                                                             for r in runs)}
            for key in ("ar_tokens_per_s", "speedup_vs_ar", "step_roofline", "kernels", "init_prefill_ms"):
                agg[key] = runs[0][key]
            extras[f"llama7b_long_w15n5g15_{mode}"] = agg
        w7 = WORKLOADS["llama7b_w7n5g7"]
        batches = {}
        for n_req in (4, 8, 16):
            log(f"llama7b_w7n5g7, {n_req} requests batched:")
            batches[str(n_req)] = measure_batch(m7, d7, w7, n_req, 256, args.warmup, args.steps)
        extras["batch_llama7b_w7n5g7"] = {
            "desc": w7["desc"] + "; n requests (prompt seeds 0..n-1) per la_batch_step under a 256-row budget, "
                                 "aggregate tokens/s, against the same requests batched autoregressively",
            "requests": batches}
        extras["tiny_w5n3g5"] = measure_tiny(args.warmup)
        line["extra_workloads"] = extras
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
