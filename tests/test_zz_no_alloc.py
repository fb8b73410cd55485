"""mk_decode_step_async_noalloc, the step for callers that cannot allocate:
its output equals mk_decode_step_async's (same kernels, same work table and
exchange layout, only the scratch memory differs), bit for bit, on calls in
a row whose inputs shrink and whose models change, so the shared static
array's parameters and tags are refreshed each time."""
import numpy as np
import pytest
import torch

import synth
from oracle.model import argmax_lowest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def native():
    from quantized_gemv_amd import native as n
    assert torch.cuda.is_available()
    return n


def _decoder(native, shape, wfmt, max_ctx, seed=0):
    d = native.Decoder(shape, wfmt, max_ctx)
    d.pack(native.master_to_device(synth.make_weights(shape, seed)))
    return d


def _both(dec, token, pos):
    """The step at `pos` through the bound scratch, then again (same token,
    same position: the cache row it writes is the same) through the static
    array; returns both (logits, next token)."""
    out = []
    for step in (dec.decode_step_async, dec.decode_step_async_noalloc):
        tok = torch.tensor([token, -7], dtype=torch.int32, device="cuda")
        lg = torch.full((dec.shape.vocab,), float("nan"), dtype=torch.float32, device="cuda")
        step(tok[0:1], pos, tok[1:2], lg)
        torch.cuda.synchronize()
        out.append((lg.cpu().numpy(), int(tok[1].item())))
    dec.check_device_error()
    return out


def _same(a, b, what):
    (la, ta), (lb, tb) = a, b
    assert ta == argmax_lowest(la) and ta >= 0, what
    assert tb == ta, (what, ta, tb)
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), (what, float(np.abs(la - lb).max()))


@pytest.mark.timeout(600)
def test_noalloc_matches_bound_scratch(native):
    big = _decoder(native, synth.QWEN3_0P6B, synth.FP8_ROW, 192)
    small = _decoder(native, synth.TINY, synth.BF16, 64)
    p_big = synth.make_prompt(synth.QWEN3_0P6B.vocab, 140, 41)
    p_small = synth.make_prompt(synth.TINY.vocab, 30, 42)
    big.prefill(p_big[:130])
    small.prefill(p_small[:25])
    # 0.6B at position 130, then the tiny decoder at 25 (a smaller model and
    # context), then the tiny decoder at 10 (a smaller context again: the
    # prompt's own token there, so the cache is unchanged), then 0.6B at 131
    _same(*_both(big, int(p_big[130]), 130), "0.6B at 130")
    _same(*_both(small, int(p_small[25]), 25), "tiny at 25")
    _same(*_both(small, int(p_small[10]), 10), "tiny at 10")
    _same(*_both(big, int(p_big[131]), 131), "0.6B at 131")
    # a chain of static steps on the device equals the bound chain
    for dec, prompt, pos0 in ((small, p_small, 26), (big, p_big, 132)):
        toks = {}
        for name in ("decode_step_async", "decode_step_async_noalloc"):
            t = torch.zeros(5, dtype=torch.int32, device="cuda")
            t[0] = int(prompt[pos0])
            for i in range(4):
                getattr(dec, name)(t[i:i + 1], pos0 + i, t[i + 1:i + 2])
            torch.cuda.synchronize()
            toks[name] = t.cpu().numpy()
        assert np.array_equal(toks["decode_step_async"], toks["decode_step_async_noalloc"]), toks
    big.close()
    small.close()


def test_noalloc_rejects_a_model_above_the_static_size(native):
    """A 0.6B-wide decoder of 64 layers needs about 46 MB of step scratch,
    more than the 32 MiB static array: refused with MK_E_UNSUPPORTED, and the
    message names both sizes; nothing is launched."""
    import dataclasses
    shape = dataclasses.replace(synth.QWEN3_0P6B, n_layers=64, vocab=4096)
    d = native.Decoder(shape, synth.BF16, 16)
    d.pack(native.master_to_device(synth.make_weights(shape, 3)))
    tok = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(native.MkError) as e:
        d.decode_step_async_noalloc(tok[0:1], 0, tok[1:2])
    assert e.value.status == native.MK_E_UNSUPPORTED
    assert "33554432" in str(e.value)
    d.close()
