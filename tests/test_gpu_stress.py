"""Race detection without a race checker (the stand-in here for the
page's compute-sanitizer racecheck, which has no ROCm counterpart here):

* the stress build (libmk_stress.so, compiled with MK_STRESS) pauses for a
  pseudo-random time, different on every run, before every exchange store
  and every courier hand-over, so producers, consumers' poll rounds and LDS
  hand-offs interleave differently each time.  A missing wait, or a value
  consumed before it is complete, would change a result.  Its logits must be
  bit-identical to the headline build's, over teacher-forced steps at the
  tiny shape (every format, with and without split attention) and at the
  0.6B shape, run three times;
* determinism of the headline build at the 0.6B shape (the page's "3
  repeated runs" for every build): three runs, identical tokens and
  bit-identical logits.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def native():
    from quantized_gemv_amd import native as n
    assert torch.cuda.is_available()
    return n


def _run(native, shape, master, wfmt, prompt, n_steps, lib=False, **kw):
    """Prefill all but the last n_steps tokens, then teacher-force those:
    the logits and fused argmax of every step, and the mean kernel time per
    step (events around each launch)."""
    d = native.Decoder(shape, wfmt, len(prompt) + 4, xray=lib, **kw)
    d.pack(native.master_to_device(master))
    d.prefill(prompt[:-n_steps])
    tok = torch.zeros(2, dtype=torch.int32, device="cuda")
    lg = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    logits, toks, ms = [], [], []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(n_steps):
        pos = len(prompt) - n_steps + i
        tok[0] = int(prompt[pos])
        e0.record()
        d.decode_step_async(tok[0:1], pos, tok[1:2], lg)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        logits.append(lg.cpu().numpy().copy())
        toks.append(int(tok[1].item()))
    d.check_device_error()
    d.close()
    _run.last_ms = float(np.mean(ms))
    return np.array(logits).view(np.uint32), toks


@pytest.mark.parametrize("wfmt,split", [(synth.BF16, 0), (synth.FP8_ROW, 16), (synth.FP4_MIX, 0),
                                        (synth.FP4_MIX, 5)])
def test_stress_build_bit_identical_tiny(native, wfmt, split):
    """Tiny decoder, 24 steps at positions 96..119; split attention from
    position 0 with `split` positions per helper (0: off)."""
    m = synth.make_weights(synth.TINY, 0)
    prompt = synth.make_prompt(synth.TINY.vocab, 120, 61)
    kw = dict(split_chunk=split, split_from=0) if split else dict(split_chunk=0)
    ref, rt = _run(native, synth.TINY, m, wfmt, prompt, 24, **kw)
    for _ in range(3):
        got, gt = _run(native, synth.TINY, m, wfmt, prompt, 24, lib="stress", **kw)
        assert gt == rt
        assert np.array_equal(got, ref)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wfmt", [synth.BF16, synth.FP8_ROW])
def test_stress_build_bit_identical_qwen3(native, wfmt):
    """The 0.6B shape in the benchmark's launch: 4 steps after a 126-token
    prompt, three stress runs against the headline build."""
    m = synth.make_weights(synth.QWEN3_0P6B, 0)
    prompt = synth.make_prompt(synth.QWEN3_0P6B.vocab, 130, 62)
    ref, rt = _run(native, synth.QWEN3_0P6B, m, wfmt, prompt, 4)
    ref_ms = _run.last_ms
    for _ in range(3):
        got, gt = _run(native, synth.QWEN3_0P6B, m, wfmt, prompt, 4, lib="stress")
        assert gt == rt
        assert np.array_equal(got, ref)
        # the pauses are there: about 0.45 ms more per step at this shape
        assert _run.last_ms > 1.3 * ref_ms, (_run.last_ms, ref_ms)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wfmt", [synth.FP8_ROW, synth.FP4_MIX])
def test_determinism_three_runs_qwen3(native, wfmt):
    """G5 at the 0.6B shape: three runs of 8 steps after a 600-token prompt
    (split attention on), identical tokens and bit-identical logits."""
    m = synth.make_weights(synth.QWEN3_0P6B, 0)
    prompt = synth.make_prompt(synth.QWEN3_0P6B.vocab, 608, 63)
    runs = [_run(native, synth.QWEN3_0P6B, m, wfmt, prompt, 8) for _ in range(3)]
    for got, gt in runs[1:]:
        assert gt == runs[0][1]
        assert np.array_equal(got, runs[0][0])
