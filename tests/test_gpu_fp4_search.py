"""GPU parity of the NVFP4 per-block MSE scale search (option 9) through the
C-ABI: the packer's bytes equal the oracle quantizer's bit for bit, and the
decode step run on the searched weights passes the op-by-op check."""
import copy

import numpy as np
import pytest
import torch

import synth
from oracle.codecs import bf16_bits_to_f32, f32_to_bf16_bits
from oracle.model import Oracle, quantize_tensor
from opcheck import Weights, check_step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def native():
    from quantized_gemv_amd import native as n
    assert torch.cuda.is_available()
    return n


@pytest.fixture(scope="module")
def master():
    return synth.make_weights(synth.TINY, 0)


@pytest.fixture(scope="module")
def planted(master):
    """The tiny master with edge blocks planted into layer 0's q: the tensor
    maximum 2.625 (ts = 2^-10 exactly), a block of 2^-7 * [1 x 15, 1.25] whose
    least-error codes tie at radius 3 (1.375 and 2.0), a zero block, and a
    block scaled by 1e-3 (subnormal scale codes, the search range clipped at
    code 0)."""
    m = copy.deepcopy(master)
    q = bf16_bits_to_f32(m.layers[0]["q"]).copy()
    assert np.abs(q).max() < 2.625
    q[0, 0] = 2.625
    q[1, 16:32] = 2.0 ** -7
    q[1, 21] = 1.25 * 2.0 ** -7
    q[2, 0:16] = 0.0
    q[3, 16:32] *= np.float32(1e-3)
    m.layers[0]["q"] = f32_to_bf16_bits(q)
    return m


def _check_fp4(codes, bs, ts, ref, what):
    assert np.array_equal(codes, ref.codes), what
    assert np.array_equal(bs, ref.block_scales), what
    assert np.float32(ts).view(np.uint32) == np.float32(ref.tensor_scale).view(np.uint32), what


@pytest.mark.parametrize("k", [1, 3, 126])
def test_searched_packed_bytes_bit_exact(native, planted, k):
    d = native.Decoder(synth.TINY, synth.FP4_MIX, 64, fp4_search=k)
    d.pack(native.master_to_device(planted))
    orc = Oracle(planted, synth.FP4_MIX, 64, fp4_search=k)
    for layer in range(synth.TINY.n_layers):
        for name in ("q", "k", "v", "o", "gate", "up"):
            codes, _, bs, ts = d.read_packed(layer, name)
            _check_fp4(codes, bs, ts, orc.packed[(layer, name)], (k, layer, name))
    codes, _, bs, ts = d.read_packed(0, "q")
    assert ts == np.float32(2.0 ** -10)
    if k == 3:
        assert bs[1, 1] == 0x3B          # the tie goes to the smaller code
    assert bs[2, 0] == 0 and np.all(codes[2, :8] == 0)
    d.close()


def test_search_changes_the_scales(native, master):
    """The search is live on the GPU: a large share of the blocks move off
    the absolute-maximum code."""
    d0 = native.Decoder(synth.TINY, synth.FP4_MIX, 64)
    d4 = native.Decoder(synth.TINY, synth.FP4_MIX, 64, fp4_search=4)
    dev = native.master_to_device(master)
    d0.pack(dev)
    d4.pack(dev)
    _, _, b0, _ = d0.read_packed(1, "gate")
    _, _, b4, _ = d4.read_packed(1, "gate")
    moved = np.mean(b0 != b4)
    assert 0.2 < moved and np.all(np.abs(b0.astype(int) - b4.astype(int)) <= 4), moved
    d0.close()
    d4.close()
    with pytest.raises(native.MkError):
        native.Decoder(synth.TINY, synth.FP4_MIX, 64, fp4_search=127)


def test_ops_tiny_searched_weights(native, master):
    """Every layer and output of a step at position 39 on weights packed
    with the search (radius 4), checked against the oracle's searched
    weights."""
    sh = synth.TINY
    toks = synth.make_prompt(sh.vocab, 40, 17)
    d = native.Decoder(sh, synth.FP4_MIX, 64, fp4_search=4)
    d.pack(native.master_to_device(master))
    d.prefill(toks[:39])
    tok = torch.tensor([int(toks[39]), 0], dtype=torch.int32, device="cuda")
    lg = torch.zeros(sh.vocab, dtype=torch.float32, device="cuda")
    d.decode_step_async(tok[0:1], 39, tok[1:2], lg)
    torch.cuda.synchronize()
    d.check_device_error()

    class Step:
        def read_exchange(self, layer, vec):
            return d.read_exchange(layer, vec)

        def kv_bits(self):
            return d.kv_cache_bits()

    check_step(Step(), Weights(master, synth.FP4_MIX, fp4_search=4), sh, int(toks[39]), 39, lg.cpu().numpy(),
               range(sh.n_layers), np.random.default_rng(0))
    d.close()


@pytest.mark.timeout(900)
def test_searched_packed_bytes_qwen3_0p6b(native):
    """At the Qwen3-0.6B shape, radius 4: four whole tensors bit-exact."""
    sh = synth.QWEN3_0P6B
    m = synth.make_weights(sh, 0)
    d = native.Decoder(sh, synth.FP4_MIX, 256, fp4_search=4)
    d.pack(native.master_to_device(m))
    for layer, name in ((0, "q"), (0, "v"), (13, "gate"), (27, "up")):
        codes, _, bs, ts = d.read_packed(layer, name)
        ref, _ = quantize_tensor(m.layers[layer][name], "fp4", 4)
        _check_fp4(codes, bs, ts, ref, (layer, name))
    d.close()
