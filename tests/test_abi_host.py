"""Host-side checks of the C-ABI library (no GPU needed).

* every function include/mk.h declares is exported by libmk.so and by the
  X-ray build;
* argument and call-order validation runs before any HIP call, so every
  error path the header documents is reachable here;
* the packed byte budget of the Qwen3-0.6B shape equals the figures the
  monolith page prints ("Upstream facts": weights read per step, 880.9 MB of
  layers plus 311.2 MB of LM head; per-layer and total weight counts; the
  FP8 and NVFP4 per-token estimates of the byte-budget block), fixture
  tests/golden/qwen3_0p6b_budget.json.
"""
import ctypes
import json
import os
import re

import numpy as np

import pytest

import synth
from quantized_gemv_amd import native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return native.load(False)


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("mk_create", "mk_query_sizes", "mk_bind", "mk_pack_weights", "mk_prefill", "mk_decode_step",
              "mk_decode_step_async", "mk_get_trace", "mk_read_packed", "mk_read_exchange", "mk_destroy"):
        assert n in names


@pytest.mark.parametrize("xray", [False, True, "stress"])
def test_library_exports_every_declared_symbol(xray):
    L = ctypes.CDLL(native.lib_path(xray))
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    assert native.load(xray).mk_has_xray() == (1 if xray is True else 0)


def _create(lib, shape=synth.TINY, wfmt=synth.BF16, max_ctx=64, **over):
    cfg = native.make_config(shape, wfmt, max_ctx)
    for k, v in over.items():
        setattr(cfg, k, v)
    h = ctypes.c_void_p()
    rc = lib.mk_create(ctypes.byref(cfg), ctypes.byref(h))
    return rc, h


def test_create_validates_the_config(lib):
    assert _create(lib)[0] == native.MK_OK
    assert _create(lib, hidden=0)[0] == native.MK_E_INVALID
    assert _create(lib, max_ctx=-1)[0] == native.MK_E_INVALID
    assert _create(lib, wfmt=7)[0] == native.MK_E_INVALID
    assert _create(lib, rms_eps=0.0)[0] == native.MK_E_INVALID
    assert _create(lib, n_kv_heads=3)[0] == native.MK_E_UNSUPPORTED       # 4 % 3 != 0
    assert _create(lib, head_dim=96)[0] == native.MK_E_UNSUPPORTED        # shape class not compiled
    assert _create(lib, max_ctx=(1 << 20) + 1)[0] == native.MK_E_UNSUPPORTED
    assert lib.mk_create(None, None) == native.MK_E_INVALID


def test_calls_out_of_order_and_bad_arguments(lib):
    rc, h = _create(lib)
    assert rc == 0
    V = synth.TINY.vocab
    # decode before bind / pack
    assert lib.mk_decode_step(h, 1, 0, None) == native.MK_E_STATE
    assert lib.mk_decode_step(h, V, 0, None) == native.MK_E_INVALID
    assert lib.mk_decode_step(h, -1, 0, None) == native.MK_E_INVALID
    assert lib.mk_decode_step(h, 1, 64, None) == native.MK_E_INVALID
    toks = (ctypes.c_int32 * 3)(1, 2, 3)
    assert lib.mk_prefill(h, toks, 3, None) == native.MK_E_STATE
    assert lib.mk_prefill(h, toks, 0, None) == native.MK_E_INVALID
    bad = (ctypes.c_int32 * 2)(1, V)
    assert lib.mk_prefill(h, bad, 2, None) == native.MK_E_INVALID
    assert lib.mk_decode_step_async(h, None, 0, None, None, None) == native.MK_E_INVALID
    assert lib.mk_decode_step_async(h, 256, 0, 256, None, None) == native.MK_E_INVALID   # same buffer
    assert lib.mk_decode_step_async(h, 256, 0, 512, None, None) == native.MK_E_STATE
    assert lib.mk_check_device_error(h, None) == native.MK_E_STATE
    # bind: null or misaligned buffers are refused before any HIP call
    assert lib.mk_bind(h, None, 256, 256, 256, None, None) == native.MK_E_INVALID
    assert lib.mk_bind(h, 256, 256, 256 + 8, 256, None, None) == native.MK_E_INVALID
    # packing before bind, wrong tensor count
    ptrs = (ctypes.c_void_p * 3)(256, 256, 256)
    assert lib.mk_pack_weights(h, ptrs, 3, None) == native.MK_E_INVALID
    n = 2 + 11 * synth.TINY.n_layers
    ptrs = (ctypes.c_void_p * n)(*([256] * n))
    assert lib.mk_pack_weights(h, ptrs, n, None) == native.MK_E_STATE
    assert lib.mk_read_packed(h, 0, 0, ctypes.c_void_p(256), None, None, None) == native.MK_E_STATE
    assert lib.mk_read_packed(h, 0, 9, ctypes.c_void_p(256), None, None, None) == native.MK_E_INVALID
    assert lib.mk_read_packed(h, 5, 0, ctypes.c_void_p(256), None, None, None) == native.MK_E_INVALID
    buf = (ctypes.c_float * synth.TINY.hidden)()
    assert lib.mk_read_exchange(h, 0, 2, buf, synth.TINY.hidden) == native.MK_E_STATE     # no step yet
    assert lib.mk_read_exchange(h, 0, 5, buf, synth.TINY.hidden) == native.MK_E_INVALID   # bad vector
    assert lib.mk_read_exchange(h, 2, 2, buf, synth.TINY.hidden) == native.MK_E_INVALID   # bad layer
    assert lib.mk_read_exchange(h, 0, 2, buf, 7) == native.MK_E_INVALID                   # wrong length
    # options
    assert lib.mk_set_option(h, 99, 0) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_GRID, -1) == native.MK_E_INVALID
    assert lib.mk_set_option(h, 1, 0) == native.MK_E_INVALID          # reserved keys
    assert lib.mk_set_option(h, 2, 64) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_POLL_SLEEP, 17) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_LAUNCH_MODE, 2) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_LAUNCH_MODE, -2) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_LAUNCH_MODE, 1) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_SPLIT_CHUNK, -1) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_SPLIT_CHUNK, 64) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_SPLIT_FROM, -3) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_SPLIT_FROM, 448) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_FP4_SEARCH, -1) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_FP4_SEARCH, 127) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_FP4_SEARCH, 126) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_FP4_SEARCH, 0) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_PREFILL_MODE, 2) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_PREFILL_MODE, -1) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_PREFILL_MODE, 1) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_PREFILL_MODE, 0) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_SYNC_MODE, 3) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_SYNC_MODE, 2) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_SYNC_MODE, -1) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_SYNC_MODE, 1) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_SYNC_MODE, 0) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_LM_BALANCE, 2) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_LM_BALANCE, -1) == native.MK_E_INVALID
    assert lib.mk_set_option(h, native.OPT_LM_BALANCE, 1) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_LM_BALANCE, 0) == native.MK_OK
    assert lib.mk_set_option(h, native.OPT_SPIN_LIMIT, 1000) == native.MK_OK
    assert lib.mk_last_error(h)
    n_out = ctypes.c_size_t(7)
    assert lib.mk_get_trace(h, None, 0, ctypes.byref(n_out)) == native.MK_OK and n_out.value == 0
    assert lib.mk_get_trace(h, None, 0, None) == native.MK_E_INVALID
    assert lib.mk_decode_codes(5, None, 0, None, None) == native.MK_E_INVALID
    assert lib.mk_decode_codes(0, None, 4, None, None) == native.MK_E_INVALID
    assert lib.mk_decode_codes(0, None, 0, None, None) == native.MK_OK      # nothing to do
    lib.mk_destroy(h)
    lib.mk_destroy(None)
    for s in range(-5, 1):
        assert lib.mk_status_str(s) != b"unknown status"


def _sizes(lib, wfmt, shape=synth.QWEN3_0P6B):
    rc, h = _create(lib, shape, wfmt, 2048)
    assert rc == 0
    s = native.mk_sizes()
    assert lib.mk_query_sizes(h, ctypes.byref(s)) == 0
    lib.mk_destroy(h)
    return s


def test_byte_budget_matches_the_page(lib):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "qwen3_0p6b_budget.json")))
    sh = synth.QWEN3_0P6B
    H, I, hd, L, V = sh.hidden, sh.intermediate, sh.head_dim, sh.n_layers, sh.vocab
    att = H * (sh.n_q_heads + 2 * sh.n_kv_heads) * hd + sh.n_q_heads * hd * H
    mlp = 3 * H * I
    assert round(att / 1e6, 2) == g["weights_per_layer_attention_M"]
    assert round(mlp / 1e6, 2) == g["weights_per_layer_mlp_M"]
    assert round((att + mlp) / 1e6, 1) == g["weights_per_layer_M"]
    assert round(L * (att + mlp) / 1e6, -1) == g["weights_layers_M"]
    assert round(V * H / 1e6, 1) == g["weights_embedding_M"]
    assert round((L * (att + mlp) + V * H) / 1e6) == g["weights_total_M"]

    bf16 = _sizes(lib, synth.BF16)
    head = V * H * 2
    layers = bf16.weight_bytes_per_token - head
    # layers include the norm gains (page: 880.9 MB of layers, 311.2 MB of LM head)
    assert round(layers / 1e6, 1) == g["bytes_layers_bf16_MB"]
    assert round(head / 1e6, 1) == g["bytes_lm_head_bf16_MB"]
    assert round(bf16.weight_bytes_per_token / 1e6, 1) == g["bytes_per_step_bf16_MB"]
    assert bf16.weight_bytes_per_token == 1_192_099_840
    fp8 = _sizes(lib, synth.FP8_ROW)
    assert fp8.weight_bytes_per_token == 598_099_456
    assert round(fp8.weight_bytes_per_token / 1e9, 2) == g["bytes_per_token_fp8_GB_approx"]
    fp4 = _sizes(lib, synth.FP4_MIX)
    assert fp4.weight_bytes_per_token == 442_697_888
    # the page's ~0.40 GB assumes down_proj in NVFP4 too; with down in FP8 the
    # difference is exactly the down matrices' FP8 minus NVFP4 bytes
    down_fp4 = H * I // 2 + H * I // 16 + 4
    down_fp8 = H * I + 4 * H
    page_mix = fp4.weight_bytes_per_token - L * (down_fp8 - down_fp4)
    assert round(page_mix / 1e9, 2) == g["bytes_per_token_nvfp4_GB_approx"]
    # KV bytes per cached position: L * 2 * nkv * hd * 2
    assert bf16.kv_bytes_per_position == L * 2 * sh.n_kv_heads * hd * 2 == 114_688


def test_kv_cache_read_back_layout():
    """The binding's KV read-back inverts the device layout mk.h states (K
    planes row-major, V planes in tiles of 4 positions, planes of max_ctx
    rounded up to 4), written here element by element from that statement."""
    import types
    import torch
    L, nkv, hd, ctx = 2, 3, 8, 6
    c4 = 8
    sh = types.SimpleNamespace(n_layers=L, n_kv_heads=nkv, head_dim=hd)
    want = np.random.default_rng(0).integers(0, 1 << 16, (L, 2, nkv, ctx, hd)).astype(np.uint16)
    flat = np.zeros(L * 2 * nkv * c4 * hd, np.uint16)
    for l in range(L):
        for kv in range(2):
            for g in range(nkv):
                base = ((l * 2 + kv) * nkv + g) * c4 * hd
                for j in range(ctx):
                    for e in range(hd):
                        off = j * hd + e if kv == 0 else (j // 4 * hd + e) * 4 + j % 4
                        flat[base + off] = want[l, kv, g, j, e]
    fake = types.SimpleNamespace(shape=sh, max_ctx=ctx, kv=torch.from_numpy(flat.view(np.uint8).copy()))
    got = native.Decoder.kv_cache_bits(fake)
    assert got.shape == want.shape and np.array_equal(got, want)
