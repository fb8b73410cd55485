"""Quantization quality on synthetic weights (oracle; test infrastructure only).

The monolith page ("Design decisions", NVFP4 format; "Measurement") asks
for the NVFP4 scales to come from a per-block search that minimizes the
squared error, and for each format's output to be compared with the bf16
model's.  Without trained weights or a dataset, both are measured here on
the seeded synthetic Qwen3-0.6B-shaped weights, with the oracle alone:

  mse     per NVFP4 matrix kind (q, k, v, o, gate, up) of the sampled layers:
          the relative squared error sum (w - w_hat)^2 / sum w^2 of the
          absolute-maximum recipe and of the search at each radius.
  logits  teacher-forced decode after the 128-token prompt: per position
          the KL divergence KL(p_bf16 || p_fmt) of the softmax distributions,
          whether the top-1 token equals bf16's, and the relative L2
          distance of the logits, for FP8 per row and FP4-mix (without and
          with the search).
  greedy  the page's first-64-token greedy agreement: per prompt, each
          format decodes 64 tokens greedily on its own; the agreement is the
          fraction of those positions whose token equals bf16's, averaged
          over the prompts.

Random weights give flat, nearly uninformative output distributions, so
these figures flag gross breakage and compare recipes on equal terms; they
say nothing of a trained model's quality.

    python -m oracle.quality [--layers 0,13,27] [--radii 1,2,4,8] [--steps 64] [--prompts 8]
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

from .codecs import bf16_bits_to_f32
from .model import Oracle
from .quant import quant_fp4

FP4_KINDS = ("q", "k", "v", "o", "gate", "up")


def relative_sq_error(w: np.ndarray, w_hat: np.ndarray) -> float:
    w64 = w.astype(np.float64)
    d = w64 - w_hat.astype(np.float64)
    return float(np.sum(d * d) / np.sum(w64 * w64))


def mse_report(master, layers, radii):
    from concurrent.futures import ThreadPoolExecutor
    jobs = [(l, kind, k) for l in layers for kind in FP4_KINDS for k in (0,) + tuple(radii)]

    def one(job):
        l, kind, k = job
        w = bf16_bits_to_f32(master.layers[l][kind])
        return job, relative_sq_error(w, quant_fp4(w, k).dequant())

    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        res = dict(ex.map(one, jobs))
    rows = []
    for kind in FP4_KINDS:
        vals = {k: float(np.mean([res[(l, kind, k)] for l in layers])) for k in (0,) + tuple(radii)}
        rows.append((kind, vals))
    tot = {k: float(np.mean([v[k] for _, v in rows])) for k in (0,) + tuple(radii)}
    return rows, tot


def softmax64(x: np.ndarray) -> np.ndarray:
    """The softmax of a logit vector, in float64."""
    z = x.astype(np.float64) - np.max(x)
    e = np.exp(z)
    return e / e.sum()


def kl_divergence(ref_logits: np.ndarray, logits: np.ndarray) -> float:
    """KL(p || q) in nats, p and q the softmax distributions of the
    reference logits and of the other logits: sum_i p_i (log p_i - log q_i),
    a term with p_i = 0 counting 0."""
    p, q = softmax64(ref_logits), softmax64(logits)
    t = np.where(p > 0, p * (np.log(np.where(p > 0, p, 1.0)) - np.log(q)), 0.0)
    return float(np.sum(t))


def greedy_agreement(ref_tokens, tokens, n: int = 64) -> float:
    """The fraction of the first n positions at which two greedy decodes of
    the same prompt chose the same token (the page's agreement measure)."""
    a, b = np.asarray(ref_tokens)[:n], np.asarray(tokens)[:n]
    if len(a) < n or len(b) < n:
        raise ValueError(f"need {n} tokens from each decode")
    return float(np.mean(a == b))


def teacher_forced_logits(master, wfmt, prompt, forced, fp4_search=0):
    orc = Oracle(master, wfmt, len(prompt) + len(forced), fp4_search=fp4_search)
    cache = orc.new_cache()
    _, last = orc.prefill_batched(cache, prompt)
    out = [last]
    for i, t in enumerate(forced[:-1]):
        out.append(orc.step(cache, int(t), len(prompt) + i))
    return np.array(out)


def logits_report(master, prompt, forced, variants):
    import synth
    ref = teacher_forced_logits(master, synth.BF16, prompt, forced)
    rows = []
    for name, wfmt, k in variants:
        got = teacher_forced_logits(master, wfmt, prompt, forced, k)
        kl, top1, rel = [], [], []
        for a, b in zip(ref, got):
            kl.append(kl_divergence(a, b))
            top1.append(int(np.argmax(a)) == int(np.argmax(b)))
            rel.append(float(np.linalg.norm(b - a) / np.linalg.norm(a)))
        rows.append((name, float(np.mean(kl)), float(np.max(kl)), float(np.mean(top1)), float(np.mean(rel))))
    return rows


def greedy_report(master, prompts, n, variants):
    """Mean first-n greedy agreement with bf16 over the prompts, per format."""
    import synth

    def decode(wfmt, k):
        orc = Oracle(master, wfmt, max(len(p) for p in prompts) + n, fp4_search=k)
        return [orc.generate(p, n - 1, batched_prefill=True)[0] for p in prompts]

    ref = decode(synth.BF16, 0)
    rows = []
    for name, wfmt, k in variants:
        got = decode(wfmt, k)
        agree = [greedy_agreement(a, b, n) for a, b in zip(ref, got)]
        distinct = np.mean([len(set(t)) for t in got])
        rows.append((name, float(np.mean(agree)), float(np.min(agree)), float(distinct)))
    return rows, float(np.mean([len(set(t)) for t in ref]))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--layers", default="0,13,27")
    ap.add_argument("--radii", default="1,2,4,8")
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--search", type=int, default=4, help="radius of the searched FP4-mix variant")
    ap.add_argument("--prompts", type=int, default=8, help="prompts of the greedy agreement")
    ap.add_argument("--greedy-len", type=int, default=64)
    args = ap.parse_args()
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import synth
    sh = synth.QWEN3_0P6B
    t0 = time.time()
    master = synth.make_weights(sh, 0)
    layers = [int(x) for x in args.layers.split(",")]
    radii = [int(x) for x in args.radii.split(",")]
    rows, tot = mse_report(master, layers, radii)
    print(f"NVFP4 relative squared error, layers {layers} (mean over layers)")
    print("| matrix | absmax | " + " | ".join(f"search k={k}" for k in radii) + " |")
    print("|---|---:|" + "---:|" * len(radii))
    for kind, v in rows + [("all kinds", tot)]:
        print(f"| {kind} | {v[0]:.5f} | " + " | ".join(f"{v[k]:.5f} ({v[k] / v[0]:.3f}x)" for k in radii) + " |")
    wl = synth.WORKLOADS["qwen3_0p6b_bf16"]
    prompt = synth.make_prompt(sh.vocab, wl.prompt_len, wl.prompt_seed)
    forced = synth.make_prompt(sh.vocab, args.steps, 21)
    variants = [("fp8 per row", synth.FP8_ROW, 0), ("fp4-mix absmax", synth.FP4_MIX, 0),
                (f"fp4-mix search k={args.search}", synth.FP4_MIX, args.search)]
    print(f"\nteacher-forced logits vs bf16, positions {wl.prompt_len - 1}..{wl.prompt_len + args.steps - 2}")
    print("| format | mean KL | max KL | top-1 = bf16 | mean rel L2 |")
    print("|---|---:|---:|---:|---:|")
    for name, kl, klmax, top1, rel in logits_report(master, prompt, forced, variants):
        print(f"| {name} | {kl:.3e} | {klmax:.3e} | {top1:.3f} | {rel:.4f} |")
    prompts = [synth.make_prompt(sh.vocab, wl.prompt_len, 100 + i) for i in range(args.prompts)]
    rows, ref_distinct = greedy_report(master, prompts, args.greedy_len, variants)
    print(f"\nfirst-{args.greedy_len}-token greedy agreement with bf16, {args.prompts} prompts of "
          f"{wl.prompt_len} tokens (bf16 itself: {ref_distinct:.1f} distinct tokens per decode)")
    print("| format | mean agreement | min agreement | distinct tokens per decode |")
    print("|---|---:|---:|---:|")
    for name, mean, low, distinct in rows:
        print(f"| {name} | {mean:.3f} | {low:.3f} | {distinct:.1f} |")
    print(f"\n({time.time() - t0:.0f} s)")


if __name__ == "__main__":
    main()
