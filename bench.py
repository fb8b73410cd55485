"""Batch-1 decode benchmark on one MI355X.

One step = one decode launch of the whole hot path (embed, 28 layers of
norm/QKV/attention/O/MLP, final norm, tied LM head, argmax) at batch 1.
Protocol (monolith page, "Hard constraints" and "Design decisions",
benchmark protocol): prefill excluded and untimed, a full warm-up pass,
re-prefill, then K greedy steps with tokens chained on the device, timed with
events around the whole loop.  Prints one JSON line.

    python bench.py [--steps 256] [--warmup 16] [--workload qwen3_0p6b_bf16]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="qwen3_0p6b_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the oracle baseline")
    ap.add_argument("--repeats", type=int, default=5, help="timed runs; the median is reported")
    ap.add_argument("--poll-sleep", type=int, default=-1, help="poll back-off 0/1 (-1: library default)")
    ap.add_argument("--launch", type=int, default=-1, help="0 cooperative, 1 plain launch (-1: library default, plain when the grid fits at once)")
    ap.add_argument("--prompt-len", type=int, default=0,
                    help="position sweep: prompt length in place of the workload's (the line then names "
                         "the workload '<name>@<prompt_len>')")
    ap.add_argument("--split-chunk", type=int, default=-1,
                    help="split attention: cached positions per workgroup (0 off, -1 library default)")
    ap.add_argument("--split-from", type=int, default=-1,
                    help="split attention from this position on (-1: library default)")
    ap.add_argument("--xray-dump", default="", help="with --xray: also save the raw records (.npy)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before decoding, run a plain device copy of this many MiB three times (the "
                         "known-size reference for scaling HBM traffic counters under rocprofv3 --pmc)")
    ap.add_argument("--prefill-bench", action="store_true",
                    help="also time mk_prefill of the workload's prompt both ways (one decode launch per "
                         "position, and the batched matrix-core prefill) and add a 'prefill' object")
    ap.add_argument("--grid", type=int, default=0, help="workgroups per launch (0: one per compute unit)")
    ap.add_argument("--one-step-per-launch", action="store_true",
                    help="time K single-step launches (mk_decode_step_async) instead of one call of K steps "
                         "(mk_decode_steps_async)")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the comparison runs of K single-step launches")
    ap.add_argument("--sync", type=int, default=0,
                    help="0 tagged exchange words (the default); 1 one grid barrier per phase hand-off with "
                         "relaxed counters; 2 the same barrier with agent-scope release/acquire fences")
    ap.add_argument("--no-fp8", action="store_true",
                    help="with the bf16 workload, skip the FP8 workload's figure that the line carries too")
    ap.add_argument("--xray", action="store_true",
                    help="X-ray build: print the per-phase budget of the step at position P + K/2 "
                         "instead of the headline line")
    return ap.parse_args()


def prefill_bench(dec, native, prompt, repeats=3):
    """Wall time of mk_prefill (synchronous) for the prompt, per path: the
    median of `repeats` runs after one untimed run."""
    res = {"prompt_len": int(len(prompt))}
    for mode, name in ((0, "decode_launches"), (1, "batched")):
        dec._check(dec.lib.mk_set_option(dec.h, native.OPT_PREFILL_MODE, mode))
        dec.prefill(prompt)
        ts = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            dec.prefill(prompt)
            ts.append(time.perf_counter() - t0)
        t = sorted(ts)[len(ts) // 2]
        res[name] = {"ms": round(t * 1e3, 3), "tokens_per_s": round(len(prompt) / t, 1)}
    dec._check(dec.lib.mk_set_option(dec.h, native.OPT_PREFILL_MODE, 0))
    return res


def xray_report(dec, wl, K, prompt, dump=""):
    """Run the X-ray build to position P + K/2 and report that step's budget."""
    import torch
    from quantized_gemv_amd import xray
    tok = torch.zeros(2, dtype=torch.int32, device="cuda")
    tok[0] = dec.prefill(prompt)
    pos = wl.prompt_len
    for i in range(K // 2):
        dec.decode_step_async(tok[i % 2:i % 2 + 1], pos + i, tok[1 - i % 2:2 - i % 2])
    torch.cuda.synchronize()
    dec.check_device_error()
    rec = dec.trace()
    if dump:
        import numpy as np
        np.save(dump, rec)
    b = xray.budget(rec, wl.shape.n_layers)
    tab = xray.phase_table(rec, wl.shape.n_layers)
    L = wl.shape.n_layers
    rnd = lambda d: {k: round(v, 1) if isinstance(v, float) else v for k, v in d.items()}
    layer_mid = {t["name"]: rnd(t) for ph, t in tab.items() if 2 <= ph < 6 * L + 2 and (ph - 2) // 6 == L // 2}
    return {"xray_position": pos + K // 2 - 1, "budget": b, "middle_layer_phases": layer_mid,
            "embed": rnd(tab.get(1, {})), "lm_head": rnd(tab.get(6 * L + 2, {})),
            "argmax": rnd(tab.get(6 * L + 3, {}))}


def kernel_source_hash() -> str:
    """sha256 over the decode kernel's sources: traffic counters taken from
    another version of the kernel are not reported."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_gemv_amd", "csrc")
    for name in ("mk_decode.hip", "mk_sync.h", "mk_shared.h", "mk_codec.h", "mk_xray.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per decode step from profiles/decode_kernel_traffic.json
    (FETCH_SIZE and WRITE_SIZE of the timed dispatches, each scaled by the
    same counter's reading for a plain copy of known size), with the
    algorithmic bytes per step of the steps they were taken over, or
    (None, None) when absent or taken on another version of the kernel."""
    path = os.path.join(ROOT, "profiles", "decode_kernel_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None, None
    e = d.get("workloads", {}).get(workload)
    if not e or d.get("kernel_source_sha256") != kernel_source_hash():
        return None, None
    return int(e["fetch_bytes_per_step"] + e["write_bytes_per_step"]), e.get("algorithmic_bytes_per_step")


def cpu_baseline(master, wl, n_steps, prompt, budget_s):
    """The oracle as it stands, timed on this host over a bounded sample of
    the timed workload: after an untimed batched prefill of the prompt, the
    decode steps at positions P..P+n_steps-1 (a second pass over the same
    positions if time is left), stopping once `budget_s` seconds of timed
    decoding have been spent."""
    import numpy as np
    from oracle.model import Oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    orc = Oracle(master, wl.wfmt, wl.prompt_len + n_steps + 1)
    done, spent, last = 0, 0.0, wl.prompt_len
    tokens, gaps = [], []   # the first pass's greedy tokens and the top-2 gap behind each
    for rep in range(2):
        cache = orc.new_cache()
        tok, lg = orc.prefill_batched(cache, prompt)
        if rep == 0:
            tokens.append(tok)
            gaps.append(top2_gap(lg))
        for i in range(n_steps):
            t0 = time.perf_counter()
            lg = orc.step(cache, tok, wl.prompt_len + i)
            tok = argmax_lowest(lg)
            spent += time.perf_counter() - t0
            done += 1
            last = max(last, wl.prompt_len + i)
            if rep == 0:
                tokens.append(tok)
                gaps.append(top2_gap(lg))
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    out = {"value": done / spent, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{done} greedy decode steps at positions {wl.prompt_len}..{last} (the timed positions, "
                     f"in up to two passes, each after an untimed batched prefill of the same "
                     f"{wl.prompt_len}-token prompt); {spent:.1f} s of numpy float32 on the host"}
    return out, tokens, gaps


# Largest logit difference between two orders of summation of the oracle
# itself (its batched against its stepwise prefill, then the same tokens) at
# the 0.6B shape after the 128-token prompt; twice it is the margin below
# which a top-2 gap counts as a near-tie (the parity tests measure it per
# step).
ORDER_NOISE = 1.5e-2


def top2_gap(logits) -> float:
    import numpy as np
    t = np.partition(logits, -2)[-2:]
    return float(t[1] - t[0])


def argmax_lowest(logits) -> int:
    import numpy as np
    return int(np.flatnonzero(logits == np.max(logits))[0])


def greedy_gate(gpu_tokens, oracle_tokens, oracle_gaps):
    """The same-session correctness gate (the page's "Hard constraints": no
    speed number counts unless that build passed the correctness check in
    the same session): the timed run's greedy tokens against the oracle's
    own greedy decode of the same prompt.  They must agree up to the first
    step whose oracle top-2 gap is below the near-tie margin; past a
    divergence the two sequences are no longer comparable."""
    n = min(len(gpu_tokens), len(oracle_tokens))
    margin = max(1e-3, 2 * ORDER_NOISE)
    agree = 0
    while agree < n and int(gpu_tokens[agree]) == int(oracle_tokens[agree]):
        agree += 1
    first_tie = next((i for i in range(n) if oracle_gaps[i] < margin), None)
    res = {"compared": n, "agree_prefix": agree, "near_tie_margin": margin, "first_near_tie": first_tie}
    if agree < n:
        res["divergence_oracle_gap"] = round(float(oracle_gaps[agree]), 6)
    # a divergence is allowed only at or after the first near-tie
    res["pass"] = bool(agree == n or (first_tie is not None and agree >= first_tie))
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this benchmark runs on one GPU only (one model replica per GPU; no multi-GPU path); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    from quantized_gemv_amd import native

    wl = synth.WORKLOADS[args.workload]
    if args.prompt_len > 0:
        import dataclasses
        wl = dataclasses.replace(wl, name=f"{wl.name}@{args.prompt_len}", prompt_len=args.prompt_len,
                                 max_ctx=args.prompt_len + args.steps + 8)
    sh = wl.shape
    K, W = args.steps, args.warmup
    max_ctx = max(wl.max_ctx, wl.prompt_len + max(K, W) + 1)
    torch.cuda.set_device(0)
    master = synth.make_weights(sh, wl.weight_seed)
    prompt = synth.make_prompt(sh.vocab, wl.prompt_len, wl.prompt_seed)

    dec = native.Decoder(sh, wl.wfmt, max_ctx, xray=args.xray, grid=args.grid, sync_mode=args.sync or None,
                         poll_sleep=None if args.poll_sleep < 0 else args.poll_sleep,
                         launch_mode=None if args.launch < 0 else args.launch,
                         split_chunk=None if args.split_chunk < 0 else args.split_chunk,
                         split_from=None if args.split_from < 0 else args.split_from)
    dev_master = native.master_to_device(master)
    dec.pack(dev_master)
    del dev_master
    torch.cuda.empty_cache()

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)   # reads and writes n*4 bytes
        torch.cuda.synchronize()
        del a, b
    if args.xray:
        print(json.dumps({"workload": wl.name, **xray_report(dec, wl, K, prompt, args.xray_dump)}), flush=True)
        dec.close()
        return
    # the same steps as K single-step launches, for comparison (not the
    # value); first, so that the timed launches are the run's last decode
    # dispatches (what the counter summaries take)
    compare = not (args.one_step_per_launch or args.no_compare)
    res1 = time_decode(dec, wl, prompt, K, W, 3, True) if compare else None
    res = time_decode(dec, wl, prompt, K, W, args.repeats, args.one_step_per_launch)
    dec.close()
    del dec
    out = {
        "metric": "batch-1 decode tokens/s (0.6B shape); % of HBM roofline on weight bytes",
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "bf16", 1: "fp8_e4m3", 2: "fp4_e2m1+fp8_e4m3"}[wl.wfmt],
        "data": "synthetic (seeded random weights N(0,0.02), uniform random prompt)",
        "config": {"workload": wl.name, "prompt_len": wl.prompt_len, "decode_steps": K,
                   "positions": [wl.prompt_len, wl.prompt_len + K - 1],
                   "weight_format": synth.WFMT_NAMES[wl.wfmt], "accumulate": "f32", "batch": 1,
                   "grid": "one workgroup per CU: 1 courier + 7 compute waves; attention on one "
                           "workgroup per KV head, split over the workgroups of its XCD from 704 "
                           "cached positions on" if not args.grid else f"{args.grid} workgroups",
                   "launch": "K single-step launches" if args.one_step_per_launch else
                             "one mk_decode_steps_async call of K steps (one launch; positions with "
                             "split-attention helpers launch one by one)",
                   "timed_runs": len(res["times"]),
                   "run_seconds": [round(t, 6) for t in res["times"]]},
        "weight_bytes_per_token": res["weight_bytes"],
        "weight_roofline_pct": res["weight_roofline_pct"],
        "roofline": res["roofline"],
        "greedy_tokens_head": [int(t) for t in res["tokens"][:8]],
    }
    if res1 is not None:
        out["one_step_per_launch"] = {"value": res1["value"], "ms_per_step": res1["ms_per_step"],
                                      "tokens_match": bool(np.array_equal(res1["tokens"], res["tokens"]))}
    if wl.name == "qwen3_0p6b_bf16" and not args.no_fp8 and args.prompt_len <= 0:
        # the FP8 workload (same master, same prompt and positions), timed the same way
        wl8 = synth.WORKLOADS["qwen3_0p6b_fp8"]
        d8 = native.Decoder(sh, wl8.wfmt, max_ctx, grid=args.grid)
        dev_master = native.master_to_device(master)
        d8.pack(dev_master)
        del dev_master
        torch.cuda.empty_cache()
        r81 = time_decode(d8, wl8, prompt, K, W, 3, True) if compare else None
        r8 = time_decode(d8, wl8, prompt, K, W, args.repeats, args.one_step_per_launch)
        d8.close()
        del d8
        out["fp8"] = {"workload": wl8.name, "value": r8["value"], "unit": "tokens/s", "ms_per_step": r8["ms_per_step"],
                      "dtype": "fp8_e4m3", "weight_bytes_per_token": r8["weight_bytes"],
                      "weight_roofline_pct": r8["weight_roofline_pct"], "roofline": r8["roofline"],
                      "run_seconds": [round(t, 6) for t in r8["times"]]}
        if r81 is not None:
            out["fp8"]["one_step_per_launch"] = {"value": r81["value"], "ms_per_step": r81["ms_per_step"],
                                                 "tokens_match": bool(np.array_equal(r81["tokens"], r8["tokens"]))}
    if args.prefill_bench:
        dp = native.Decoder(sh, wl.wfmt, max_ctx, grid=args.grid)
        dp.pack(native.master_to_device(master))
        out["prefill"] = prefill_bench(dp, native, prompt)
        dp.close()
    if not args.no_cpu_baseline:
        cpu, o_tokens, o_gaps = cpu_baseline(master, wl, K, prompt, args.cpu_seconds)
        out["cpu_baseline"] = cpu
        out["greedy_gate"] = greedy_gate(res["tokens"], o_tokens, o_gaps)
    torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


def time_decode(dec, wl, prompt, K, W, repeats, one_per_launch=False):
    """W untimed warm-up steps, then `repeats` timed runs of K steps, each
    after an untimed prefill: HIP events on the stream the kernel runs on
    around one mk_decode_steps_async call of K steps (one launch; with
    one_per_launch, K chained single-step launches).  Returns the median
    figures."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    toks = torch.zeros(max(K, W) + 1, dtype=torch.int32, device="cuda")

    def run(n):
        first = dec.prefill(prompt)
        toks[0] = first
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if one_per_launch:
            for i in range(n):
                dec.decode_step_async(toks[i:i + 1], wl.prompt_len + i, toks[i + 1:i + 2])
        else:
            dec.decode_steps_async(toks[0:1], wl.prompt_len, n, toks[1:n + 1])
        e1.record(stream)
        torch.cuda.synchronize()
        dec.check_device_error()
        return e0.elapsed_time(e1) / 1e3

    run(W)                       # warm-up pass
    times = [run(K) for _ in range(max(1, repeats))]
    tokens = toks[:K + 1].cpu().numpy().copy()
    dt = float(np.median(times))
    tps = K / dt
    sizes = dec.sizes
    wbytes = int(sizes.weight_bytes_per_token)
    # algorithmic bytes per launch: every weight byte once, plus the KV cache
    # read over positions 0..pos (mean over the timed positions)
    mean_ctx = wl.prompt_len + (K - 1) / 2.0 + 1
    algo = wbytes + float(sizes.kv_bytes_per_position) * mean_ctx   # per step
    achieved = algo / (dt / K) / 1e9
    spl = 1 if one_per_launch else K   # steps per launch
    # the counters were taken over the 256 timed steps of the default run
    # (positions P..P+255, one launch); their ratio to those steps'
    # algorithmic bytes is what a reader compares, whatever window this run
    # timed
    traffic, traffic_algo = measured_traffic(wl.name)
    return {"value": round(tps, 2), "ms_per_step": round(dt / K * 1e3, 5), "times": times, "tokens": tokens,
            "weight_bytes": wbytes, "weight_roofline_pct": round(100.0 * wbytes * tps / (PEAK_HBM_GBPS * 1e9), 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(achieved / PEAK_HBM_GBPS, 4),
                         "traffic": int(traffic * spl) if traffic else None,
                         "traffic_over_algorithmic": round(traffic / traffic_algo, 4) if traffic and traffic_algo else None,
                         "traffic_window": f"the 256 steps at positions {wl.prompt_len}..{wl.prompt_len + 255}"
                                           if traffic else None,
                         "kernel": "mk::decode_kernel", "steps_per_launch": spl,
                         "bytes_per_launch": int(algo * spl), "launch_us": round(dt / K * spl * 1e6, 2)}}


if __name__ == "__main__":
    main()
