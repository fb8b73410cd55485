"""Pins of the op-by-op checker (tests/opcheck.py) on the CPU: it accepts
the oracle's own intermediates, and it rejects each of a set of plausible
kernel mistakes planted into them (a dropped product term, a sign error, a
skipped or missing attention position, a wrong rotation, swapped pairs, a
1e-3 scale error)."""
import numpy as np
import pytest

import synth
from oracle.codecs import bf16_round, f32_to_bf16_bits
from oracle.model import Oracle, apply_rope, argmax_lowest, gqa_attention, rmsnorm, rope_table
from opcheck import Weights, check_step

SH = synth.TINY


class OracleStep:
    """The intermediates of one oracle step, in the form check_step reads."""

    def __init__(self, trace, cache):
        self.t = trace
        self.kv = np.stack([f32_to_bf16_bits(cache.k.astype(np.float32)),
                            f32_to_bf16_bits(cache.v.astype(np.float32))], axis=1)

    def read_exchange(self, layer, vec):
        return np.asarray(self.t[(layer, vec)], dtype=np.float32).copy()

    def kv_bits(self):
        return self.kv


@pytest.fixture(scope="module")
def master():
    return synth.make_weights(SH, 0)


def _run(master, wfmt, pos, seed=5):
    toks = synth.make_prompt(SH.vocab, pos + 1, seed)
    orc = Oracle(master, wfmt, pos + 8)
    cache = orc.new_cache()
    orc.prefill_batched(cache, toks[:pos])
    trace = {}
    logits = orc.step(cache, int(toks[pos]), pos, trace=trace)
    return orc, cache, trace, logits, int(toks[pos])


@pytest.mark.parametrize("wfmt,pos", [(synth.BF16, 20), (synth.FP8_ROW, 20), (synth.FP4_MIX, 20),
                                      (synth.BF16, 450)])
def test_accepts_the_oracles_own_step(master, wfmt, pos):
    orc, cache, trace, logits, tok = _run(master, wfmt, pos)
    check_step(OracleStep(trace, cache), Weights(master, wfmt), SH, tok, pos, logits, range(SH.n_layers),
               np.random.default_rng(0))
    # and with sampled rows
    check_step(OracleStep(trace, cache), Weights(master, wfmt), SH, tok, pos, logits, range(SH.n_layers),
               np.random.default_rng(1), n_sample=24)


def _attention(orc, trace, cache, l, pos, keep):
    """The attention output of layer l over the cached positions in `keep`."""
    nq, nkv, hd = SH.n_q_heads, SH.n_kv_heads, SH.head_dim
    cos, sin = rope_table(pos + 1, hd, SH.rope_theta)
    qraw = trace[(l, "qkv")][:nq * hd].reshape(nq, hd)
    q = apply_rope(rmsnorm(qraw, orc.w[l]["q_norm"], SH.rms_eps), cos[pos], sin[pos])
    return bf16_round(gqa_attention(q, cache.k[l][:, keep], cache.v[l][:, keep]).reshape(-1))


MISTAKES = ["o_dropped_term", "k_output_sign", "attn_skips_a_position", "attn_without_current",
            "v_append_off_by_one_ulp", "k_append_rotation_sign", "swiglu_pairs_swapped", "down_scale",
            "lm_head_row"]


@pytest.mark.parametrize("mistake", MISTAKES)
def test_rejects_planted_mistakes(master, mistake):
    pos, l = 30, 1
    orc, cache, trace, logits, tok = _run(master, synth.BF16, pos)
    nq, nkv, hd = SH.n_q_heads, SH.n_kv_heads, SH.head_dim
    expect = None
    if mistake == "o_dropped_term":
        o = trace[(l, "attn")]
        j = 7
        terms = orc.w[l]["o"][j] * o
        i = int(np.argmax(np.abs(terms)))
        trace[(l, "x_o")][j] -= terms[i]
        expect = "o_proj"
    elif mistake == "k_output_sign":
        trace[(l, "qkv")][nq * hd + 3] *= -1
        expect = "'k'"
    elif mistake == "attn_skips_a_position":
        keep = [p for p in range(pos + 1) if p != pos // 2]
        trace[(l, "attn")] = _attention(orc, trace, cache, l, pos, keep)
        expect = "attention"
    elif mistake == "attn_without_current":
        trace[(l, "attn")] = _attention(orc, trace, cache, l, pos, list(range(pos)))
        expect = "attention"
    elif mistake == "v_append_off_by_one_ulp":
        row = cache.v[l, 0, pos].astype(np.float32)
        bits = f32_to_bf16_bits(row)
        bits[5] += 1
        from oracle.codecs import bf16_bits_to_f32
        cache.v[l, 0, pos] = bf16_bits_to_f32(bits)
        expect = "V append"
    elif mistake == "k_append_rotation_sign":
        cos, sin = rope_table(pos + 1, hd, SH.rope_theta)
        kraw = trace[(l, "qkv")][nq * hd:(nq + nkv) * hd].reshape(nkv, hd)
        k = apply_rope(rmsnorm(kraw, orc.w[l]["k_norm"], SH.rms_eps), cos[pos], -sin[pos])
        cache.k[l, :, pos] = bf16_round(k)
        expect = "K append"
    elif mistake == "swiglu_pairs_swapped":
        h = trace[(l, "h")]
        trace[(l, "h")] = h.reshape(-1, 2)[:, ::-1].reshape(-1).copy()
        expect = "swiglu"
    elif mistake == "down_scale":
        trace[(l, "x_d")] = trace[(l, "x_d")] * np.float32(1.001)
        expect = "down"
    elif mistake == "lm_head_row":
        logits = logits.copy()
        logits[argmax_lowest(logits)] += np.float32(1e-3) * np.abs(logits).max()
        expect = "lm_head"
    with pytest.raises(AssertionError) as e:
        check_step(OracleStep(trace, cache), Weights(master, synth.BF16), SH, tok, pos, logits,
                   range(SH.n_layers), np.random.default_rng(0))
    assert expect in str(e.value), str(e.value)[:300]
