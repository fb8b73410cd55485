"""Op-by-op GPU parity through the C-ABI.

After a decode step, every phase's output is read back (mk_read_exchange and
the caller-owned KV cache) and recomputed by tests/opcheck.py with the
oracle's functions from the GPU's own input to that phase (tolerances there).

Tiny decoder: every layer and every output.  Qwen3-0.6B shape, launched as
the benchmark launches it (one workgroup per compute unit): a sample of
layers and of output rows, at the benchmark's first timed position and at
positions whose attention streams cache passes beyond the ones held in
registers.
"""
import numpy as np
import pytest
import torch

import synth
from oracle.model import Oracle, argmax_lowest
from opcheck import Weights, check_step

pytestmark = pytest.mark.gpu

FORMATS = [synth.BF16, synth.FP8_ROW, synth.FP4_MIX]


@pytest.fixture(scope="module")
def native():
    from quantized_gemv_amd import native as n
    assert torch.cuda.is_available()
    return n


class GpuStep:
    """The intermediates of the decoder's last step, for check_step."""

    def __init__(self, dec, sh):
        self.dec, self.sh = dec, sh

    def read_exchange(self, layer, vec):
        return self.dec.read_exchange(layer, vec)

    def kv_bits(self):
        return self.dec.kv_cache_bits()


def _step(dec, sh, token, pos):
    tok = torch.tensor([token, 0], dtype=torch.int32, device="cuda")
    lg = torch.zeros(sh.vocab, dtype=torch.float32, device="cuda")
    dec.decode_step_async(tok[0:1], pos, tok[1:2], lg)
    torch.cuda.synchronize()
    dec.check_device_error()
    logits = lg.cpu().numpy()
    assert int(tok[1].item()) == argmax_lowest(logits)
    return logits


def _decoder(native, shape, master, wfmt, max_ctx, **kw):
    d = native.Decoder(shape, wfmt, max_ctx, **kw)
    d.pack(native.master_to_device(master))
    return d


# ------------------------------------------------------------------ tiny
@pytest.fixture(scope="module")
def tiny_master():
    return synth.make_weights(synth.TINY, 0)


@pytest.mark.parametrize("wfmt", FORMATS)
def test_ops_tiny_every_output(native, tiny_master, wfmt):
    """All layers, all outputs, at position 39 (after a 39-token prefill)."""
    sh = synth.TINY
    toks = synth.make_prompt(sh.vocab, 40, 11)
    d = _decoder(native, sh, tiny_master, wfmt, 64)
    d.prefill(toks[:39])
    logits = _step(d, sh, int(toks[39]), 39)
    check_step(GpuStep(d, sh), Weights(tiny_master, wfmt), sh, int(toks[39]), 39, logits, range(sh.n_layers),
               np.random.default_rng(0))
    d.close()


def test_ops_tiny_streamed_attention(native, tiny_master):
    """Positions 470 and 700 without split attention: one and three cache
    passes stream after the four held in registers (max_ctx 702, not a
    multiple of the 4-position V tile)."""
    sh = synth.TINY
    toks = synth.make_prompt(sh.vocab, 701, 12)
    d = _decoder(native, sh, tiny_master, synth.BF16, 702, split_chunk=0)
    W = Weights(tiny_master, synth.BF16)
    d.prefill(toks[:470])
    logits = _step(d, sh, int(toks[470]), 470)
    check_step(GpuStep(d, sh), W, sh, int(toks[470]), 470, logits, range(sh.n_layers), np.random.default_rng(0))
    for pos in range(471, 700):
        _step(d, sh, int(toks[pos]), pos)
    logits = _step(d, sh, int(toks[700]), 700)
    check_step(GpuStep(d, sh), W, sh, int(toks[700]), 700, logits, range(sh.n_layers), np.random.default_rng(0))
    d.close()


@pytest.mark.parametrize("wfmt,chunk,positions", [
    (synth.BF16, 8, (39,)),             # 4 helpers per head, slices of 8
    (synth.FP4_MIX, 5, (39,)),          # 7 helpers, one-wave slices
    (synth.FP8_ROW, 16, (400, 470)),    # 25 and all 31 helpers, streamed home slice
    (synth.BF16, 1, (470,)),            # every helper, slices of 15
])
def test_ops_tiny_split_attention(native, tiny_master, wfmt, chunk, positions):
    """Split attention: the head's positions spread over its home and
    helper workgroups, partials merged by the home; every output checked."""
    sh = synth.TINY
    n = max(positions) + 1
    toks = synth.make_prompt(sh.vocab, n, 14)
    d = _decoder(native, sh, tiny_master, wfmt, n + 8, split_chunk=chunk, split_from=0)
    W = Weights(tiny_master, wfmt)
    d.prefill(toks[:positions[0]])
    for pos in range(positions[0], n):
        logits = _step(d, sh, int(toks[pos]), pos)
        if pos in positions:
            check_step(GpuStep(d, sh), W, sh, int(toks[pos]), pos, logits, range(sh.n_layers),
                       np.random.default_rng(pos))
    d.close()


@pytest.mark.parametrize("split", [0, 16])
def test_ops_tiny_block_boundaries(native, tiny_master, split):
    """Every output of every layer at the positions where the attention's
    block structure changes: position 0 (no cached position), the ends of the
    first 16-position block and of the first pass of 7 blocks (112), the end
    of the held range (448 = 4 passes) and the first streamed pass; with the
    home workgroup alone and with helpers taking slices of 16 (split attention
    from position 0, slice boundaries inside blocks)."""
    sh = synth.TINY
    positions = (0, 1, 15, 16, 17, 111, 112, 113, 447, 448, 449)
    n = positions[-1] + 1
    toks = synth.make_prompt(sh.vocab, n, 18)
    d = _decoder(native, sh, tiny_master, synth.FP8_ROW, n + 3, split_chunk=split, split_from=0)
    W = Weights(tiny_master, synth.FP8_ROW)
    for pos in range(n):
        logits = _step(d, sh, int(toks[pos]), pos)
        if pos in positions:
            check_step(GpuStep(d, sh), W, sh, int(toks[pos]), pos, logits, range(sh.n_layers),
                       np.random.default_rng(pos))
    d.close()


def test_split_attention_deterministic(native, tiny_master):
    """The split path's merge order is fixed: two runs, identical bits."""
    sh = synth.TINY
    toks = synth.make_prompt(sh.vocab, 120, 15)
    outs = []
    for _ in range(2):
        d = _decoder(native, sh, tiny_master, synth.FP8_ROW, 128, split_chunk=4, split_from=0)
        d.prefill(toks[:100])
        got = [_step(d, sh, int(toks[pos]), pos).view(np.uint32).copy() for pos in range(100, 120)]
        outs.append(np.array(got))
        d.close()
    assert np.array_equal(outs[0], outs[1])


def test_exchange_needs_a_step(native, tiny_master):
    d = _decoder(native, synth.TINY, tiny_master, synth.BF16, 64)
    with pytest.raises(native.MkError):
        d.read_exchange(0, "x_o")
    d.close()


# ------------------------------------------------------------ Qwen3-0.6B
@pytest.fixture(scope="module")
def q_master():
    return synth.make_weights(synth.QWEN3_0P6B, 0)


Q_LAYERS = (0, 1, 14, 27)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wfmt", FORMATS)
def test_ops_qwen3_0p6b_sampled(native, q_master, wfmt):
    """The benchmark's workload and launch: the 128-token prompt, then the
    first timed step (position 128); layers 0, 1, 14, 27 and the LM head,
    160 sampled rows of every matrix (plus the first, the last and the
    argmax row)."""
    sh = synth.QWEN3_0P6B
    wl = {synth.BF16: "qwen3_0p6b_bf16", synth.FP8_ROW: "qwen3_0p6b_fp8",
          synth.FP4_MIX: "qwen3_0p6b_fp4mix"}[wfmt]
    prompt = synth.make_prompt(sh.vocab, 128, synth.WORKLOADS[wl].prompt_seed)
    d = _decoder(native, sh, q_master, wfmt, 512)
    first = d.prefill(prompt)
    logits = _step(d, sh, first, 128)
    check_step(GpuStep(d, sh), Weights(q_master, wfmt), sh, first, 128, logits, Q_LAYERS, np.random.default_rng(1),
               n_sample=160)
    d.close()


@pytest.mark.timeout(900)
def test_ops_qwen3_0p6b_streamed_attention(native, q_master):
    """Positions 460 and 600 without split attention (one and two streamed
    cache passes), bf16."""
    sh = synth.QWEN3_0P6B
    toks = synth.make_prompt(sh.vocab, 601, 13)
    d = _decoder(native, sh, q_master, synth.BF16, 640, split_chunk=0)
    W = Weights(q_master, synth.BF16)
    d.prefill(toks[:460])
    logits = _step(d, sh, int(toks[460]), 460)
    check_step(GpuStep(d, sh), W, sh, int(toks[460]), 460, logits, Q_LAYERS, np.random.default_rng(2), n_sample=96)
    for pos in range(461, 600):
        _step(d, sh, int(toks[pos]), pos)
    logits = _step(d, sh, int(toks[600]), 600)
    check_step(GpuStep(d, sh), W, sh, int(toks[600]), 600, logits, Q_LAYERS, np.random.default_rng(3), n_sample=96)
    d.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wfmt,chunk", [(synth.BF16, 16), (synth.FP8_ROW, 4)])
def test_ops_qwen3_0p6b_split_attention(native, q_master, wfmt, chunk):
    """Split attention at the 0.6B shape: position 128 after the benchmark's
    prompt (8 or all 31 helpers per head) and position 460."""
    sh = synth.QWEN3_0P6B
    wl = synth.WORKLOADS["qwen3_0p6b_bf16"]
    prompt = synth.make_prompt(sh.vocab, wl.prompt_len, wl.prompt_seed)
    toks = np.concatenate([prompt, synth.make_prompt(sh.vocab, 340, 16)])
    d = _decoder(native, sh, q_master, wfmt, 512, split_chunk=chunk, split_from=0)
    W = Weights(q_master, wfmt)
    d.prefill(prompt)
    for pos in range(128, 461):
        logits = _step(d, sh, int(toks[pos]), pos)
        if pos in (128, 460):
            check_step(GpuStep(d, sh), W, sh, int(toks[pos]), pos, logits, Q_LAYERS,
                       np.random.default_rng(pos), n_sample=96)
    d.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("prefill_mode", [0, 1])
def test_end_to_end_qwen3_0p6b_bf16(native, q_master, prefill_mode):
    """Whole-step parity at the benchmark's size: after the benchmark's
    prompt (mk_prefill as one decode launch per position, or the batched
    matrix-core prefill), 8 teacher-forced steps (positions 128..135) against
    the full oracle: logits within relative L2 1e-2, and the fused argmax by
    the G3 rule of tests/gates.py.  The oracle's reference is its stepwise
    prefill; its batched prefill (another summation order) gives the margin.
    With the batched GPU prefill, step 1 here is a near-tie (oracle gap
    2.8e-3 against an order noise of 1.3e-2): a token that differs there is
    a valid argmax, not a failure."""
    from gates import check_token, rel_l2
    sh = synth.QWEN3_0P6B
    wl = synth.WORKLOADS["qwen3_0p6b_bf16"]
    prompt = synth.make_prompt(sh.vocab, wl.prompt_len, wl.prompt_seed)
    orc = Oracle(q_master, synth.BF16, 160)
    cache, twin_cache = orc.new_cache(), orc.new_cache()
    _, last = orc.prefill(cache, prompt)
    _, twin = orc.prefill_batched(twin_cache, prompt)
    d = _decoder(native, sh, q_master, synth.BF16, 160, prefill_mode=prefill_mode)
    check_token(d.prefill(prompt), last, np.abs(last - twin).max(), "prefill")
    forced = synth.make_prompt(sh.vocab, 8, 21)
    for i, t in enumerate(forced):
        pos = wl.prompt_len + i
        logits = _step(d, sh, int(t), pos)
        ref, tw = orc.step(cache, int(t), pos), orc.step(twin_cache, int(t), pos)
        assert rel_l2(logits, ref) <= 1e-2, pos
        check_token(argmax_lowest(logits), ref, np.abs(ref - tw).max(), pos)
    d.close()
