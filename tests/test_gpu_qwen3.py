"""Whole-step parity at the Qwen3-0.6B shape for every benchmarked
configuration, through the C-ABI, in the benchmark's launch (one workgroup
per compute unit, library defaults):

* G1: every packed matrix of the FP8 and FP4-mix models, the tied
  embedding / LM head included, bit-exact against the oracle's quantizer;
* G2 / G3 / G4 under teacher forcing after the FP8 workload's 128-token
  prompt and the FP4-mix workload's 512-token prompt;
* free-running greedy decode (bf16, FP8) equal to the oracle's up to the
  first near-tie;
* the default split attention (from 704 cached positions) at positions 720
  and 1000, the ends of the page's position sweep (16 and 2048), and the
  long-context workload itself (FP8, 16,384-token prompt), every phase
  recomputed from the GPU's own inputs (tests/opcheck.py).

The G3 margin is the one tests/gates.py states: max(1e-3, twice the
oracle's own summation-order noise at that step)."""
import numpy as np
import pytest
import torch

import synth
from gates import REL_L2, check_token, margin, rel_l2, top2_gap
from opcheck import Weights, check_step
from oracle.model import Oracle, argmax_lowest

pytestmark = pytest.mark.gpu

SH = synth.QWEN3_0P6B
Q_LAYERS = (0, 1, 14, 27)


@pytest.fixture(scope="module")
def native():
    from quantized_gemv_amd import native as n
    assert torch.cuda.is_available()
    return n


@pytest.fixture(scope="module")
def q_master():
    return synth.make_weights(SH, 0)


def _decoder(native, master, wfmt, max_ctx, **kw):
    d = native.Decoder(SH, wfmt, max_ctx, **kw)
    d.pack(native.master_to_device(master))
    return d


def _step(dec, token, pos):
    """One step through mk_decode_step_async; returns (logits, fused argmax),
    and checks G4 (the fused argmax is the brute-force argmax of the
    logits)."""
    tok = torch.tensor([token, 0], dtype=torch.int32, device="cuda")
    lg = torch.zeros(SH.vocab, dtype=torch.float32, device="cuda")
    dec.decode_step_async(tok[0:1], pos, tok[1:2], lg)
    torch.cuda.synchronize()
    dec.check_device_error()
    logits = lg.cpu().numpy()
    fused = int(tok[1].item())
    assert fused == argmax_lowest(logits), pos
    return logits, fused


class GpuStep:
    def __init__(self, dec):
        self.dec = dec

    def read_exchange(self, layer, vec):
        return self.dec.read_exchange(layer, vec)

    def kv_bits(self):
        return self.dec.kv_cache_bits()


def _check_packed(codes, sc, bs, ts, ref, what):
    if isinstance(ref, np.ndarray):
        assert np.array_equal(codes, ref), what
    elif hasattr(ref, "scales"):
        assert np.array_equal(codes, ref.codes), what
        assert np.array_equal(sc.view(np.uint32), ref.scales.view(np.uint32)), what
    else:
        assert np.array_equal(codes, ref.codes), what
        assert np.array_equal(bs, ref.block_scales), what
        assert np.float32(ts).view(np.uint32) == np.float32(ref.tensor_scale).view(np.uint32), what


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wfmt", [synth.FP8_ROW, synth.FP4_MIX])
def test_packed_bytes_full_model(native, q_master, wfmt):
    """G1 at full size: all 197 matrices (7 per layer and the 151,936-row
    tied embedding / LM head) as the benchmark packs them."""
    d = _decoder(native, q_master, wfmt, 16)
    orc = Oracle(q_master, wfmt, 16)
    n = 0
    for layer in range(SH.n_layers):
        for name in ("q", "k", "v", "o", "gate", "up", "down"):
            _check_packed(*d.read_packed(layer, name), orc.packed[(layer, name)], (wfmt, layer, name))
            n += 1
    _check_packed(*d.read_packed(0, "embed"), orc.packed[(-1, "embed")], (wfmt, "embed"))
    assert n + 1 == 197
    d.close()


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("workload", ["qwen3_0p6b_fp8", "qwen3_0p6b_fp4mix"])
def test_teacher_forced_qwen3(native, q_master, workload):
    """G2/G3/G4 for the FP8 (128-token prompt) and FP4-mix (512-token
    prompt) workloads: the prefill's token, then 6 teacher-forced steps
    against the full oracle.  The oracle runs twice, stepwise (the reference)
    and with its batched prefill (the noise probe for the G3 margin)."""
    wl = synth.WORKLOADS[workload]
    P, n = wl.prompt_len, 6
    prompt = synth.make_prompt(SH.vocab, P, wl.prompt_seed)
    forced = synth.make_prompt(SH.vocab, n, 21)
    orc = Oracle(q_master, wl.wfmt, P + n + 1)
    ca, cb = orc.new_cache(), orc.new_cache()
    _, last = orc.prefill(ca, prompt)
    _, twin = orc.prefill_batched(cb, prompt)
    d = _decoder(native, q_master, wl.wfmt, P + n + 8)
    check_token(d.prefill(prompt), last, np.abs(last - twin).max(), (workload, "prefill"))
    strict, worst = 0, 0.0
    for i, t in enumerate(forced):
        pos = P + i
        logits, fused = _step(d, int(t), pos)
        ref, twin = orc.step(ca, int(t), pos), orc.step(cb, int(t), pos)
        r = rel_l2(logits, ref)
        worst = max(worst, r)
        assert r <= REL_L2, (workload, pos, r)
        strict += check_token(fused, ref, np.abs(ref - twin).max(), (workload, pos))
    print(f"{workload}: max rel L2 {worst:.2e}, {strict}/{n} steps decided by the strict rule")
    d.close()


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("wfmt", [synth.BF16, synth.FP8_ROW])
def test_free_running_greedy_qwen3(native, q_master, wfmt):
    """G3 free-running at the benchmark's prompt: the GPU's greedy tokens
    (mk_prefill, then mk_decode_step on its own tokens) equal the oracle's
    up to the first step whose oracle top-2 gap is below the margin."""
    wl = synth.WORKLOADS["qwen3_0p6b_bf16"]
    P, n = wl.prompt_len, 16
    prompt = synth.make_prompt(SH.vocab, P, wl.prompt_seed)
    orc = Oracle(q_master, wfmt, P + n + 1)
    ca, cb = orc.new_cache(), orc.new_cache()
    tok, last = orc.prefill(ca, prompt)
    _, twin = orc.prefill_batched(cb, prompt)
    want, gates = [tok], [(last, np.abs(last - twin).max())]
    for i in range(n):
        a, b = orc.step(ca, want[-1], P + i), orc.step(cb, want[-1], P + i)
        want.append(argmax_lowest(a))
        gates.append((a, np.abs(a - b).max()))
    d = _decoder(native, q_master, wfmt, P + n + 8)
    got = [d.prefill(prompt)]
    for i in range(n):
        got.append(d.decode_step(got[-1], P + i))
    d.close()
    compared = 0
    for i in range(n + 1):
        ref, noise = gates[i]
        if top2_gap(ref) < margin(noise):
            break
        assert got[i] == want[i], (wfmt, i, got[: i + 1], want[: i + 1])
        compared += 1
    assert compared >= 1
    print(f"wfmt {wfmt}: {compared} of {n + 1} greedy tokens compared before the first near-tie")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wfmt", [synth.FP4_MIX, synth.FP8_ROW])
def test_split_attention_default_qwen3(native, q_master, wfmt):
    """The library's default split attention at the FP4-mix workload's
    positions: at 720 (3 helpers per KV head, slices of 180 positions: two
    passes per helper) and 1000 (5 helpers, slices of 167), every phase of
    layers 0, 1, 14, 27 and the LM head recomputed from the GPU's inputs."""
    toks = synth.make_prompt(SH.vocab, 1001, 17)
    d = _decoder(native, q_master, wfmt, 1024)
    W = Weights(q_master, wfmt)
    d.prefill(toks[:720])
    for pos in range(720, 1001):
        logits, _ = _step(d, int(toks[pos]), pos)
        if pos in (720, 1000):
            check_step(GpuStep(d), W, SH, int(toks[pos]), pos, logits, Q_LAYERS, np.random.default_rng(pos),
                       n_sample=96)
    d.close()


@pytest.mark.timeout(900)
def test_long_context_fp8_16k(native, q_master):
    """The long-context workload: the FP8 model, a 16,384-token prompt run
    through mk_prefill (one decode launch per position: split attention from
    704 on), then the first decode step at position 16,384 (31 helpers per KV
    head, slices of 512 positions: five passes each), every phase of layers
    0, 1, 14, 27 and the LM head recomputed from the GPU's own cache and
    inputs."""
    wl = synth.WORKLOADS["qwen3_0p6b_fp8_long"]
    P = wl.prompt_len
    prompt = synth.make_prompt(SH.vocab, P, wl.prompt_seed)
    d = _decoder(native, q_master, synth.FP8_ROW, wl.max_ctx)
    first = d.prefill(prompt)
    logits, _ = _step(d, first, P)
    check_step(GpuStep(d), Weights(q_master, synth.FP8_ROW), SH, first, P, logits, Q_LAYERS,
               np.random.default_rng(5), n_sample=96)
    d.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wfmt,pos", [(synth.BF16, 16), (synth.BF16, 2048), (synth.FP4_MIX, 2048)])
def test_sweep_positions_qwen3(native, q_master, wfmt, pos):
    """The ends of the page's position sweep (16 and 2048 cached positions)
    not covered above, in the launch the sweep times: every phase of layers
    0, 1, 14, 27 and the LM head recomputed from the GPU's own inputs."""
    toks = synth.make_prompt(SH.vocab, pos + 1, 19)
    d = _decoder(native, q_master, wfmt, pos + 8)
    d.prefill(toks[:pos])
    logits, _ = _step(d, int(toks[pos]), pos)
    check_step(GpuStep(d), Weights(q_master, wfmt), SH, int(toks[pos]), pos, logits, Q_LAYERS,
               np.random.default_rng(pos), n_sample=96)
    d.close()
