"""Pins for the oracle's decode step: identities of each primitive, special
cases, and the whole step against the transformers library's Qwen3 model
in float64 (no GPU)."""
import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import model as M
from oracle.codecs import bf16_bits_to_f32, bf16_round

F64 = np.float64


def test_rmsnorm_identities():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1024)
    g1 = np.ones(1024)
    # scale invariance with eps = 0
    a = M.rmsnorm(x, g1, 0.0, F64)
    assert np.allclose(M.rmsnorm(37.5 * x, g1, 0.0, F64), a, rtol=1e-13, atol=0)
    # unit gains: mean(y^2) = ms / (ms + eps)
    eps = 0.3
    ms = np.mean(x * x)
    assert np.isclose(np.mean(M.rmsnorm(x, g1, eps, F64) ** 2), ms / (ms + eps), rtol=1e-13)
    # gains multiply elementwise
    g = rng.standard_normal(1024)
    assert np.allclose(M.rmsnorm(x, g, eps, F64), g * M.rmsnorm(x, g1, eps, F64), rtol=1e-13)


def test_rope_identities():
    hd, theta = 128, 1e6
    cos, sin = M.rope_table(4096, hd, theta)
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    # position 0 is the identity
    assert np.array_equal(M.apply_rope(q, cos[0], sin[0], F64), q)
    # complex form: (x_i + i x_{i+hd/2}) * exp(i p theta^(-2i/hd)), frequency 0 is 1 rad/pos
    p = 1234
    z = (q[:64] + 1j * q[64:]) * np.exp(1j * p * theta ** (-np.arange(64) / 64.0))
    r = M.apply_rope(q, cos[p].astype(F64), sin[p].astype(F64), F64)
    assert np.allclose(r, np.concatenate([z.real, z.imag]), atol=2e-7 * np.abs(q).max())
    assert cos[1, 0] == np.float32(np.cos(1.0)) and sin[1, 0] == np.float32(np.sin(1.0))
    # pair norms are preserved and scores depend only on the offset
    assert np.allclose(np.hypot(r[:64], r[64:]), np.hypot(q[:64], q[64:]), rtol=1e-6)
    d1 = M.apply_rope(q, cos[700], sin[700], F64) @ M.apply_rope(k, cos[500], sin[500], F64)
    d2 = M.apply_rope(q, cos[3200], sin[3200], F64) @ M.apply_rope(k, cos[3000], sin[3000], F64)
    assert np.isclose(d1, d2, rtol=1e-5, atol=1e-5)


def test_softmax_rows():
    rng = np.random.default_rng(2)
    s = (rng.standard_normal((64, 1000)) * 5).astype(np.float32)
    p = M.softmax(s)
    assert np.all(np.abs(p.sum(axis=1, dtype=F64) - 1) <= 1000 * 2.0 ** -24)
    assert np.allclose(M.softmax(s + np.float32(17.0)), p, rtol=1e-5, atol=1e-9)
    assert np.all(p > 0)


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    nq, nkv, hd = 16, 8, 128
    q = rng.standard_normal((nq, hd)).astype(np.float32)
    # one position: every head returns exactly its KV head's value vector
    k1 = rng.standard_normal((nkv, 1, hd)).astype(np.float32)
    v1 = rng.standard_normal((nkv, 1, hd)).astype(np.float32)
    o = M.gqa_attention(q, k1, v1)
    for h in range(nq):
        assert np.array_equal(o[h], v1[h // 2, 0])
    # zero keys: uniform weights, the output is the mean of the values
    v = rng.standard_normal((nkv, 50, hd)).astype(np.float32)
    o = M.gqa_attention(q, np.zeros((nkv, 50, hd), np.float32), v)
    for h in range(nq):
        assert np.allclose(o[h], v[h // 2].mean(axis=0), rtol=1e-5, atol=1e-6)


def test_silu_and_argmax():
    z = np.linspace(-30, 30, 6001)
    assert M.silu(np.zeros(3), F64).tolist() == [0, 0, 0]
    assert np.allclose(M.silu(z, F64), z * scipy.special.expit(z), rtol=1e-13, atol=1e-300)
    assert abs(M.silu(np.array([40.0]), F64)[0] - 40.0) < 1e-12
    rng = np.random.default_rng(4)
    for _ in range(200):
        a = rng.integers(0, 5, 50).astype(np.float32)      # many ties
        assert M.argmax_lowest(a) == min(i for i in range(50) if a[i] == a.max())


def _oracle(shape, wfmt, max_ctx=64, **kw):
    master = synth.make_weights(shape, 0)
    return master, M.Oracle(master, wfmt, max_ctx, **kw)


def _hf_model(master, o):
    from transformers import Qwen3Config, Qwen3ForCausalLM
    sh = master.shape
    cfg = Qwen3Config(vocab_size=sh.vocab, hidden_size=sh.hidden, intermediate_size=sh.intermediate,
                      num_hidden_layers=sh.n_layers, num_attention_heads=sh.n_q_heads,
                      num_key_value_heads=sh.n_kv_heads, head_dim=sh.head_dim,
                      rms_norm_eps=sh.rms_eps, rope_theta=sh.rope_theta, tie_word_embeddings=True,
                      max_position_embeddings=4096, attention_bias=False, hidden_act="silu",
                      use_sliding_window=False)
    cfg._attn_implementation = "eager"
    m = Qwen3ForCausalLM(cfg).to(torch.float64).eval()
    t = lambda a: torch.from_numpy(np.asarray(a, F64))
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(t(o.embed))
        m.model.norm.weight.copy_(t(o.final_norm))
        for l, layer in enumerate(m.model.layers):
            w = o.w[l]
            a, mlp = layer.self_attn, layer.mlp
            a.q_proj.weight.copy_(t(w["q"])); a.k_proj.weight.copy_(t(w["k"]))
            a.v_proj.weight.copy_(t(w["v"])); a.o_proj.weight.copy_(t(w["o"]))
            a.q_norm.weight.copy_(t(w["q_norm"])); a.k_norm.weight.copy_(t(w["k_norm"]))
            layer.input_layernorm.weight.copy_(t(w["in_norm"]))
            layer.post_attention_layernorm.weight.copy_(t(w["post_norm"]))
            mlp.gate_proj.weight.copy_(t(w["gate"])); mlp.up_proj.weight.copy_(t(w["up"]))
            mlp.down_proj.weight.copy_(t(w["down"]))
    assert m.lm_head.weight.data_ptr() == m.model.embed_tokens.weight.data_ptr()
    return m


@pytest.mark.parametrize("wfmt", [synth.BF16, synth.FP8_ROW, synth.FP4_MIX])
def test_step_matches_transformers_qwen3(wfmt):
    """The oracle in float64 without rounding points equals the library's
    Qwen3 decoder (same dequantized weights) run over the whole sequence."""
    master, o = _oracle(synth.TINY, wfmt, dtype=F64, round_bf16=False)
    toks = synth.make_prompt(synth.TINY.vocab, 24, seed=9)
    m = _hf_model(master, o)
    with torch.no_grad():
        ref = m(torch.from_numpy(toks.astype(np.int64))[None]).logits[0].numpy()
    cache = o.new_cache()
    for p, tk in enumerate(toks):
        lg = o.step(cache, int(tk), p)
        err = np.linalg.norm(lg - ref[p]) / np.linalg.norm(ref[p])
        assert err < 1e-5, (p, err)   # the library takes RoPE angles in float32


def test_rounding_contract_within_parity_tolerance():
    """float32 with the bf16 rounding points vs float64 without them: the
    rounding contract alone stays well inside a 1e-2 relative L2."""
    master = synth.make_weights(synth.TINY, 0)
    o32 = M.Oracle(master, synth.BF16, 64)
    o64 = M.Oracle(master, synth.BF16, 64, dtype=F64, round_bf16=False)
    toks = synth.make_prompt(synth.TINY.vocab, 40, seed=10)
    c32, c64 = o32.new_cache(), o64.new_cache()
    worst = 0.0
    for p, tk in enumerate(toks):
        a, b = o32.step(c32, int(tk), p), o64.step(c64, int(tk), p)
        worst = max(worst, np.linalg.norm(a - b) / np.linalg.norm(b))
    assert worst < 1e-2


def test_zero_layers_reduce_to_tied_embedding():
    """All layer linears zero: every residual update is 0, so the logits are
    E_hat . bf16(rmsnorm(E_hat[t], g_f))."""
    master = synth.make_weights(synth.TINY, 0, zero_linears=True)
    o = M.Oracle(master, synth.BF16, 16)
    e = bf16_bits_to_f32(master.embed)
    gf = bf16_bits_to_f32(master.final_norm)
    cache = o.new_cache()
    for p, t in enumerate([5, 4095, 0]):
        x = e[t].astype(F64)
        xf = bf16_round((gf * (x / np.sqrt(np.mean(x * x) + 1e-6))).astype(np.float32))
        ref = e.astype(F64) @ xf.astype(F64)
        got = o.step(cache, t, p)
        assert np.allclose(got, ref, rtol=1e-5, atol=1e-6)
        assert M.argmax_lowest(got) == t     # the token's own row dominates


def test_batched_prefill_equals_stepwise():
    master = synth.make_weights(synth.TINY, 0)
    toks = synth.make_prompt(synth.TINY.vocab, 20, seed=11)
    for wfmt in (synth.BF16, synth.FP4_MIX):
        o = M.Oracle(master, wfmt, 32, dtype=F64, round_bf16=False)
        c1, c2 = o.new_cache(), o.new_cache()
        n1, l1 = o.prefill(c1, toks)
        n2, l2 = o.prefill_batched(c2, toks)
        assert n1 == n2
        assert np.allclose(l1, l2, rtol=1e-10, atol=1e-12)
        assert np.allclose(c1.k, c2.k, rtol=1e-10, atol=1e-12)


# the bf16 rounding points of one layer in the batched prefill, in the order
# it takes them (GEMV input, K, V, attention output, post-attention GEMV
# input, SwiGLU output), then the final norm's output
ROUNDING_POINTS = ("xn", "k", "v", "o", "xn2", "h", "final")


def _prefill_skipping(o, toks, skip):
    """The batched prefill with rounding point `skip` (an index into
    ROUNDING_POINTS) left out in every layer: a planted mistake."""
    L = o.shape.n_layers
    orig, calls = M.Oracle._r, [0]

    def r(self, x):
        i = calls[0]
        calls[0] += 1
        hit = i % 6 == skip if i < 6 * L else skip == 6
        return x.astype(self.dt) if hit else orig(self, x)

    c = o.new_cache()
    M.Oracle._r = r
    try:
        _, logits = o.prefill_batched(c, toks)
    finally:
        M.Oracle._r = orig
    assert calls[0] == 6 * L + 1
    return c, logits


@pytest.mark.parametrize("wfmt", [synth.BF16, synth.FP8_ROW, synth.FP4_MIX])
def test_batched_prefill_rounding_points(wfmt):
    """The batched prefill takes every bf16 rounding point of the stepwise
    decode.  In float64 a change of summation order moves a value by about
    1e-16 of itself, far too little to move any float32 or bf16 rounding, so
    with the rounding points on, the batched and stepwise prefills must give
    bit-identical caches and logits.  Leaving out any one rounding point of
    the batched prefill (each planted in turn) breaks that."""
    master = synth.make_weights(synth.TINY, 0)
    toks = synth.make_prompt(synth.TINY.vocab, 48, seed=31)
    o = M.Oracle(master, wfmt, 64, dtype=F64)
    a, b = o.new_cache(), o.new_cache()
    ta, la = o.prefill(a, toks)
    tb, lb = o.prefill_batched(b, toks)
    assert ta == tb
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert np.array_equal(la, lb)
    for skip, name in enumerate(ROUNDING_POINTS):
        c, lc = _prefill_skipping(o, toks, skip)
        same = np.array_equal(a.k, c.k) and np.array_equal(a.v, c.v) and np.array_equal(la, lc)
        assert not same, ("planted mistake not caught", name)


@pytest.mark.parametrize("wfmt", [synth.BF16, synth.FP8_ROW, synth.FP4_MIX])
def test_batched_prefill_float32(wfmt):
    """In float32 (the arithmetic of the references the GPU tests use) the
    batched and stepwise prefills differ only by summation order: both
    caches hold bf16 values; layer 0, where both start from the same
    embeddings, is within one bf16 step per element and at least 99.9 %
    bit-equal; every cached row of every layer is within relative L2 1e-2;
    the logits too."""
    from oracle.codecs import bf16_round
    master = synth.make_weights(synth.TINY, 0)
    toks = synth.make_prompt(synth.TINY.vocab, 48, seed=31)
    o = M.Oracle(master, wfmt, 64)
    a, b = o.new_cache(), o.new_cache()
    _, la = o.prefill(a, toks)
    _, lb = o.prefill_batched(b, toks)
    for x, y in ((a.k, b.k), (a.v, b.v)):
        x, y = x[:, :, :48], y[:, :, :48]
        assert np.array_equal(bf16_round(y), y) and np.array_equal(bf16_round(x), x)
        x64, y64 = x.astype(F64), y.astype(F64)
        step = 2.0 ** -7 * np.maximum(np.abs(x64[0]), np.abs(y64[0]))
        assert np.all(np.abs(x64[0] - y64[0]) <= step)
        assert np.mean(x[0] == y[0]) >= 0.999
        rel = np.linalg.norm(x64 - y64, axis=-1) / np.linalg.norm(x64, axis=-1)
        assert rel.max() <= 1e-2
    assert np.linalg.norm(la - lb) / np.linalg.norm(la) <= 1e-2


def test_step_rejects_out_of_range():
    _, o = _oracle(synth.TINY, synth.BF16, max_ctx=8)
    c = o.new_cache()
    with pytest.raises(ValueError):
        o.step(c, 0, 8)
    with pytest.raises(ValueError):
        o.step(c, synth.TINY.vocab, 0)
