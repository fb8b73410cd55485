"""Several greedy steps per launch (mk_decode_steps_async; monolith page,
Part 2, "Mission": one persistent kernel per token, and its benchmark's
greedy loop).

A launch of n steps must give each step exactly what n single-step launches
give, each started on the previous one's token: identical tokens and
bit-identical logits.  The steps' tokens and logits also pass the oracle's
gates (G2 logits, G3 tokens) teacher-forced along the same tokens.  Cases
cover every weight format, the grid-barrier variants, a run that crosses
into split attention (those positions get single-step launches), the
512-step launch cap, the stress build (random pauses before every exchange
store, so workgroups drift apart across step boundaries), and the two
failure paths: a token outside the vocabulary and waits forced to time out.
"""
import numpy as np
import pytest
import torch

import synth
from gates import REL_L2, check_token, rel_l2
from oracle.model import Oracle

pytestmark = pytest.mark.gpu

FORMATS = [synth.BF16, synth.FP8_ROW, synth.FP4_MIX]


@pytest.fixture(scope="module")
def native():
    from quantized_gemv_amd import native as n
    assert torch.cuda.is_available()
    return n


@pytest.fixture(scope="module")
def master():
    return synth.make_weights(synth.TINY, 0)


def _decoder(native, shape, master, wfmt, max_ctx, **kw):
    d = native.Decoder(shape, wfmt, max_ctx, **kw)
    d.pack(native.master_to_device(master))
    return d


def _chained(d, first, pos, n, vocab):
    """n single-step launches, each reading the token the previous one wrote."""
    tok = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    tok[0] = first
    lg = torch.zeros(n, vocab, dtype=torch.float32, device="cuda")
    for i in range(n):
        d.decode_step_async(tok[i:i + 1], pos + i, tok[i + 1:i + 2], lg[i])
    torch.cuda.synchronize()
    d.check_device_error()
    return tok[1:].cpu().numpy(), lg.cpu().numpy()


def _multi(d, first, pos, n, vocab):
    tok = torch.tensor([first], dtype=torch.int32, device="cuda")
    nxt = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    lg = torch.zeros(n, vocab, dtype=torch.float32, device="cuda")
    d.decode_steps_async(tok, pos, n, nxt, lg)
    torch.cuda.synchronize()
    d.check_device_error()
    return nxt.cpu().numpy(), lg.cpu().numpy()


def _same(a, b):
    (ta, la), (tb, lb) = a, b
    assert np.array_equal(ta, tb), (ta, tb)
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))


def _oracle_gates(master, wfmt, max_ctx, prompt, first, toks, logits):
    """Teacher-forced along the GPU's own tokens: G2 on every step's logits
    and G3 on every step's token."""
    orc = Oracle(master, wfmt, max_ctx)
    cache = orc.new_cache()
    want, _ = orc.prefill(cache, prompt)
    assert first == want
    tok = first
    for i in range(len(toks)):
        ref = orc.step(cache, tok, len(prompt) + i)
        assert rel_l2(logits[i], ref) <= REL_L2, (wfmt, i)
        check_token(int(toks[i]), ref, what=(wfmt, i))
        tok = int(toks[i])


@pytest.mark.parametrize("wfmt", FORMATS)
@pytest.mark.parametrize("case", ["plain", "split", "bar1", "bar2"])
def test_steps_equal_chained_steps_tiny(native, master, wfmt, case):
    """20 steps after a 24-token prompt.  split: helpers from position 30
    (5 positions each), so one launch runs positions 24..29 and the rest run
    one per launch; bar1 and bar2: the grid-barrier variants."""
    kw = {"plain": {}, "split": dict(split_chunk=5, split_from=30),
          "bar1": dict(sync_mode=1), "bar2": dict(sync_mode=2)}[case]
    prompt = synth.make_prompt(synth.TINY.vocab, 24, 71)
    runs = []
    for fn in (_chained, _multi):
        d = _decoder(native, synth.TINY, master, wfmt, 64, **kw)
        first = d.prefill(prompt)
        runs.append(fn(d, first, 24, 20, synth.TINY.vocab))
        d.close()
    _same(runs[1], runs[0])
    _oracle_gates(master, wfmt, 64, prompt, first, *runs[1])


def test_steps_launch_cap_and_split_boundary_tiny(native, master):
    """720 steps after an 8-token prompt with the default split attention
    (helpers from position 704): launches of 512 steps (8..519) and 184
    steps (520..703), then one launch per position."""
    prompt = synth.make_prompt(synth.TINY.vocab, 8, 72)
    runs = []
    for fn in (_chained, _multi):
        d = _decoder(native, synth.TINY, master, synth.FP8_ROW, 736)
        first = d.prefill(prompt)
        runs.append(fn(d, first, 8, 720, synth.TINY.vocab))
        d.close()
    _same(runs[1], runs[0])


def test_steps_stress_build_tiny(native, master):
    """The stress build's multi-step launch against the headline build's
    single steps, three runs (split attention on from position 36)."""
    prompt = synth.make_prompt(synth.TINY.vocab, 24, 73)
    kw = dict(split_chunk=5, split_from=36)
    d = _decoder(native, synth.TINY, master, synth.FP4_MIX, 64, **kw)
    first = d.prefill(prompt)
    ref = _chained(d, first, 24, 24, synth.TINY.vocab)
    d.close()
    for _ in range(3):
        d = _decoder(native, synth.TINY, master, synth.FP4_MIX, 64, xray="stress", **kw)
        assert d.prefill(prompt) == first
        _same(_multi(d, first, 24, 24, synth.TINY.vocab), ref)
        d.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wfmt", [synth.BF16, synth.FP8_ROW])
def test_steps_lm_balance_qwen3(native, wfmt):
    """Option 12 on (LM-head rows moved between workgroups from step to
    step): 24 steps after a 64-token prompt at the 0.6B shape, bit-identical
    to single-step launches (which workgroup computes a row changes no
    result)."""
    m = synth.make_weights(synth.QWEN3_0P6B, 0)
    prompt = synth.make_prompt(synth.QWEN3_0P6B.vocab, 64, 76)
    d = _decoder(native, synth.QWEN3_0P6B, m, wfmt, 96)
    first = d.prefill(prompt)
    ref = _chained(d, first, 64, 24, synth.QWEN3_0P6B.vocab)
    d.close()
    d = _decoder(native, synth.QWEN3_0P6B, m, wfmt, 96, lm_balance=1)
    assert d.prefill(prompt) == first
    _same(_multi(d, first, 64, 24, synth.QWEN3_0P6B.vocab), ref)
    d.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wfmt,plen,n", [(synth.BF16, 64, 12), (synth.FP8_ROW, 698, 10)])
def test_steps_equal_chained_steps_qwen3(native, wfmt, plen, n):
    """The 0.6B shape: 12 bf16 steps after a 64-token prompt, and 10 FP8
    steps from position 698 (six in one launch, then split attention from
    704 one launch per position)."""
    m = synth.make_weights(synth.QWEN3_0P6B, 0)
    prompt = synth.make_prompt(synth.QWEN3_0P6B.vocab, plen, 74)
    d = _decoder(native, synth.QWEN3_0P6B, m, wfmt, plen + n + 4)
    first = d.prefill(prompt)
    ref = _chained(d, first, plen, n, synth.QWEN3_0P6B.vocab)
    d.close()
    d = _decoder(native, synth.QWEN3_0P6B, m, wfmt, plen + n + 4)
    assert d.prefill(prompt) == first
    _same(_multi(d, first, plen, n, synth.QWEN3_0P6B.vocab), ref)
    d.close()


def test_steps_invalid_token_and_arguments(native, master):
    d = _decoder(native, synth.TINY, master, synth.BF16, 64)
    tok = torch.tensor([synth.TINY.vocab + 3], dtype=torch.int32, device="cuda")
    nxt = torch.zeros(5, dtype=torch.int32, device="cuda")
    d.decode_steps_async(tok, 0, 5, nxt)
    torch.cuda.synchronize()
    assert nxt.tolist() == [-1] * 5
    with pytest.raises(native.MkError) as e:
        d.check_device_error()
    assert e.value.status == native.MK_E_INVALID
    # refused before any launch: no steps, positions past the cache or
    # negative, the input token inside the output array
    tok[0] = 1
    for src, pos, n in [(tok, 0, 0), (tok, 60, 5), (tok, -1, 2), (nxt[2:3], 0, 5)]:
        with pytest.raises(native.MkError) as e:
            d.decode_steps_async(src, pos, n, nxt)
        assert e.value.status == native.MK_E_INVALID
    d.close()


def test_steps_timeout_forced_from_host(native, master):
    """Every wait made unsatisfiable (tag skew) with a 100 us spin bound: the
    launch stops at its first step, every d_next is -1 and the device error
    is MK_E_TIMEOUT; with the hook off the same call gives the chained
    steps' results."""
    prompt = synth.make_prompt(synth.TINY.vocab, 16, 75)
    d = _decoder(native, synth.TINY, master, synth.BF16, 64)
    first = d.prefill(prompt)
    d.set_option(native.OPT_SPIN_LIMIT, 10_000)
    d.set_option(native.OPT_TAG_SKEW, 1)
    tok = torch.tensor([first], dtype=torch.int32, device="cuda")
    nxt = torch.zeros(4, dtype=torch.int32, device="cuda")
    d.decode_steps_async(tok, 16, 4, nxt)
    torch.cuda.synchronize()
    assert nxt.tolist() == [-1] * 4
    with pytest.raises(native.MkError) as e:
        d.check_device_error()
    assert e.value.status == native.MK_E_TIMEOUT
    d.set_option(native.OPT_TAG_SKEW, 0)
    d.set_option(native.OPT_SPIN_LIMIT, 100_000_000)
    got = _multi(d, first, 16, 8, synth.TINY.vocab)
    d.close()
    d = _decoder(native, synth.TINY, master, synth.BF16, 64)
    assert d.prefill(prompt) == first
    _same(got, _chained(d, first, 16, 8, synth.TINY.vocab))
    d.close()
