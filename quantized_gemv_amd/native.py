"""ctypes binding of libmk (include/mk.h), with the same names.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of the library.  PyTorch is used to allocate the device buffers the
library asks for and to supply the current HIP stream.  The library must have
been built in-tree (quantized_gemv_amd/build.py); a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

from .build import lib_path

MK_OK, MK_E_INVALID, MK_E_UNSUPPORTED, MK_E_STATE, MK_E_HIP, MK_E_TIMEOUT = 0, -1, -2, -3, -4, -5
BF16, FP8_ROW, FP4_MIX = 0, 1, 2
MATRICES = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "embed": 7}
# mk_read_exchange vectors: q/k/v GEMV outputs, attention output, residual after O, SwiGLU output,
# residual after down
EXCHANGE = {"qkv": 0, "attn": 1, "x_o": 2, "h": 3, "x_d": 4}
OPT_GRID, OPT_SPIN_LIMIT, OPT_TAG_SKEW, OPT_POLL_SLEEP, OPT_LAUNCH_MODE, OPT_SPLIT_CHUNK, OPT_SPLIT_FROM = \
    0, 3, 4, 5, 6, 7, 8
OPT_FP4_SEARCH = 9
OPT_PREFILL_MODE = 10
OPT_SYNC_MODE = 11   # 0 tagged exchange words; 1, 2 one grid barrier per phase hand-off (2: with L2 fences)
OPT_LM_BALANCE = 12  # several steps per launch: 1 LM-head rows balanced across XCDs, 0 equal shares (default)


class MkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"mk status {status}: {msg}")
        self.status = status


class mk_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("wfmt", ctypes.c_int32)]


class mk_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("weights", "kv", "rope", "scratch", "trace",
                                               "weight_bytes_per_token", "kv_bytes_per_position")]


# One X-ray record (mk_trace_rec in include/mk.h, 88 bytes).
TRACE_DTYPE = np.dtype([(n, np.uint32) for n in ("phase", "wg", "hw_id", "xcc", "active", "pad")] +
                       [(n, np.uint64) for n in ("t_start", "t_ready", "t_handoff", "t_seen", "t_done")] +
                       [("t_mark", np.uint64, (3,))])

_LIBS: Dict[object, ctypes.CDLL] = {}
_VP = ctypes.c_void_p


def load(xray=False) -> ctypes.CDLL:
    """Load libmk.so, or with xray=True libmk_xray.so, or with xray="stress"
    libmk_stress.so (MK_LIBRARY / MK_LIBRARY_XRAY name another build of the
    first two).  Raises if it has not been built."""
    if xray in _LIBS:
        return _LIBS[xray]
    env = {False: "MK_LIBRARY", True: "MK_LIBRARY_XRAY"}.get(xray)
    path = (os.environ.get(env) if env else None) or lib_path(xray)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with quantized_gemv_amd/build.py "
                           "(there is no fallback path)")
    L = ctypes.CDLL(path)
    P = ctypes.POINTER
    sig = {
        "mk_create": (ctypes.c_int, [P(mk_config), P(_VP)]),
        "mk_query_sizes": (ctypes.c_int, [_VP, P(mk_sizes)]),
        "mk_bind": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP]),
        "mk_pack_weights": (ctypes.c_int, [_VP, P(_VP), ctypes.c_int32, _VP]),
        "mk_read_packed": (ctypes.c_int, [_VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP,
                                          P(ctypes.c_float)]),
        "mk_read_exchange": (ctypes.c_int, [_VP, ctypes.c_int32, ctypes.c_int32, P(ctypes.c_float),
                                            ctypes.c_size_t]),
        "mk_prefill": (ctypes.c_int32, [_VP, P(ctypes.c_int32), ctypes.c_int32, _VP]),
        "mk_decode_step": (ctypes.c_int32, [_VP, ctypes.c_int32, ctypes.c_int32, _VP]),
        "mk_decode_step_async": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, _VP, _VP, _VP]),
        "mk_decode_step_async_noalloc": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, _VP, _VP, _VP]),
        "mk_decode_steps_async": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP]),
        "mk_check_device_error": (ctypes.c_int, [_VP, _VP]),
        "mk_get_trace": (ctypes.c_int, [_VP, _VP, ctypes.c_size_t, P(ctypes.c_size_t)]),
        "mk_decode_codes": (ctypes.c_int, [ctypes.c_int32, _VP, ctypes.c_int32, _VP, _VP]),
        "mk_set_option": (ctypes.c_int, [_VP, ctypes.c_int32, ctypes.c_int64]),
        "mk_has_xray": (ctypes.c_int, []),
        "mk_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "mk_last_error": (ctypes.c_char_p, [_VP]),
        "mk_destroy": (None, [_VP]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _LIBS[xray] = L
    return L


def make_config(shape, wfmt: int, max_ctx: int) -> mk_config:
    return mk_config(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                     shape.intermediate, shape.vocab, max_ctx, shape.rope_theta, shape.rms_eps, wfmt)


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Decoder:
    """One model handle with its device buffers (allocated through torch)."""

    def __init__(self, shape, wfmt: int, max_ctx: int, xray=False, grid: int = 0,
                 spin_limit: Optional[int] = None, poll_sleep: Optional[int] = None,
                 launch_mode: Optional[int] = None, split_chunk: Optional[int] = None,
                 split_from: Optional[int] = None, fp4_search: Optional[int] = None,
                 prefill_mode: Optional[int] = None, sync_mode: Optional[int] = None,
                 lm_balance: Optional[int] = None):
        import torch
        self.lib = load(xray)
        self.shape, self.wfmt, self.max_ctx = shape, wfmt, max_ctx
        self.cfg = make_config(shape, wfmt, max_ctx)
        h = _VP()
        self._check(self.lib.mk_create(ctypes.byref(self.cfg), ctypes.byref(h)), None)
        self.h = h
        if grid:
            self._check(self.lib.mk_set_option(self.h, OPT_GRID, grid))
        if spin_limit is not None:
            self._check(self.lib.mk_set_option(self.h, OPT_SPIN_LIMIT, spin_limit))
        if poll_sleep is not None:
            self._check(self.lib.mk_set_option(self.h, OPT_POLL_SLEEP, poll_sleep))
        if launch_mode is not None:
            self._check(self.lib.mk_set_option(self.h, OPT_LAUNCH_MODE, launch_mode))
        if split_chunk is not None:
            self._check(self.lib.mk_set_option(self.h, OPT_SPLIT_CHUNK, split_chunk))
        if split_from is not None:
            self._check(self.lib.mk_set_option(self.h, OPT_SPLIT_FROM, split_from))
        if fp4_search is not None:
            self._check(self.lib.mk_set_option(self.h, OPT_FP4_SEARCH, fp4_search))
        if prefill_mode is not None:
            self._check(self.lib.mk_set_option(self.h, OPT_PREFILL_MODE, prefill_mode))
        if sync_mode is not None:
            self._check(self.lib.mk_set_option(self.h, OPT_SYNC_MODE, sync_mode))
        if lm_balance is not None:
            self._check(self.lib.mk_set_option(self.h, OPT_LM_BALANCE, lm_balance))
        self.sizes = mk_sizes()
        self._check(self.lib.mk_query_sizes(self.h, ctypes.byref(self.sizes)))
        dev = torch.device("cuda", torch.cuda.current_device())
        alloc = lambda n: torch.empty(max(int(n), 256), dtype=torch.uint8, device=dev)
        self.weights = alloc(self.sizes.weights)
        self.kv = alloc(self.sizes.kv)
        self.rope = alloc(self.sizes.rope)
        self.scratch = alloc(self.sizes.scratch)
        self.trace_buf = alloc(self.sizes.trace) if self.sizes.trace else None
        self._check(self.lib.mk_bind(self.h, self.weights.data_ptr(), self.kv.data_ptr(), self.rope.data_ptr(),
                                     self.scratch.data_ptr(),
                                     self.trace_buf.data_ptr() if self.trace_buf is not None else None,
                                     _stream()))

    def _check(self, rc: int, h=-1):
        if rc < 0:
            hh = self.h if h == -1 else h
            msg = self.lib.mk_last_error(hh).decode() if hh else self.lib.mk_status_str(rc).decode()
            raise MkError(rc, msg)
        return rc

    def set_option(self, key: int, value: int):
        self._check(self.lib.mk_set_option(self.h, key, value))

    def pack(self, tensors: Sequence) -> None:
        """`tensors`: the 2 + 11*L bf16 device tensors in the mk_pack_weights order."""
        ptrs = (_VP * len(tensors))(*[t.data_ptr() for t in tensors])
        self._check(self.lib.mk_pack_weights(self.h, ptrs, len(tensors), _stream()))

    def read_packed(self, layer: int, matrix: str):
        """Canonical packed form of one matrix: (codes, scales, block_scales, tensor_scale)."""
        sh = self.shape
        H, I, hd = sh.hidden, sh.intermediate, sh.head_dim
        NK = {"q": (sh.n_q_heads * hd, H), "k": (sh.n_kv_heads * hd, H), "v": (sh.n_kv_heads * hd, H),
              "o": (H, sh.n_q_heads * hd), "gate": (I, H), "up": (I, H), "down": (H, I),
              "embed": (sh.vocab, H)}[matrix]
        N, K = NK
        fmt = _tensor_format(self.wfmt, matrix)
        if fmt == "bf16":
            codes = np.empty((N, K), np.uint16)
        elif fmt == "fp8":
            codes = np.empty((N, K), np.uint8)
        else:
            codes = np.empty((N, K // 2), np.uint8)
        scales = np.empty(N, np.float32)
        bscales = np.empty((N, K // 16), np.uint8)
        ts = ctypes.c_float(0.0)
        self._check(self.lib.mk_read_packed(self.h, layer, MATRICES[matrix], codes.ctypes.data,
                                            scales.ctypes.data, bscales.ctypes.data, ctypes.byref(ts)))
        return codes, (scales if fmt == "fp8" else None), (bscales if fmt == "fp4" else None), \
            (np.float32(ts.value) if fmt == "fp4" else None)

    def read_exchange(self, layer: int, vec: str) -> np.ndarray:
        """The last step's activation `vec` of `layer` (see EXCHANGE)."""
        sh = self.shape
        n = {"qkv": (sh.n_q_heads + 2 * sh.n_kv_heads) * sh.head_dim, "attn": sh.n_q_heads * sh.head_dim,
             "x_o": sh.hidden, "h": sh.intermediate, "x_d": sh.hidden}[vec]
        out = np.empty(n, np.float32)
        self._check(self.lib.mk_read_exchange(self.h, layer, EXCHANGE[vec],
                                              out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), n))
        return out

    def kv_cache_bits(self) -> np.ndarray:
        """The KV cache as bf16 bit patterns [n_layers, 2, n_kv_heads, max_ctx,
        head_dim] (K then V), read back from the device layout mk.h states:
        planes of ctx4 = max_ctx rounded up to 4 positions, K row-major, V in
        tiles of 4 positions."""
        sh = self.shape
        c4 = (self.max_ctx + 3) & ~3
        n = sh.n_layers * 2 * sh.n_kv_heads * c4 * sh.head_dim
        raw = self.kv[: 2 * n].cpu().numpy().view(np.uint16).reshape(sh.n_layers, 2, sh.n_kv_heads, c4 * sh.head_dim)
        k = raw[:, 0].reshape(sh.n_layers, sh.n_kv_heads, c4, sh.head_dim)
        v = raw[:, 1].reshape(sh.n_layers, sh.n_kv_heads, c4 // 4, sh.head_dim, 4).transpose(0, 1, 2, 4, 3)
        v = v.reshape(sh.n_layers, sh.n_kv_heads, c4, sh.head_dim)
        return np.stack([k, v], axis=1)[:, :, :, : self.max_ctx].copy()

    def prefill(self, tokens: Sequence[int]) -> int:
        arr = (ctypes.c_int32 * len(tokens))(*[int(t) for t in tokens])
        return self._check(self.lib.mk_prefill(self.h, arr, len(tokens), _stream()))

    def decode_step(self, token: int, pos: int) -> int:
        return self._check(self.lib.mk_decode_step(self.h, int(token), int(pos), _stream()))

    def decode_step_async(self, d_token, pos: int, d_next, d_logits=None) -> None:
        self._check(self.lib.mk_decode_step_async(self.h, d_token.data_ptr(), int(pos), d_next.data_ptr(),
                                                  d_logits.data_ptr() if d_logits is not None else None,
                                                  _stream()))

    def decode_steps_async(self, d_token, pos: int, n: int, d_next, d_logits=None) -> None:
        """mk_decode_steps_async: n greedy steps from position pos; d_next
        (int32[n]) receives each step's token, d_logits (fp32 [n][vocab]) if
        given each step's logits."""
        self._check(self.lib.mk_decode_steps_async(self.h, d_token.data_ptr(), int(pos), int(n), d_next.data_ptr(),
                                                   d_logits.data_ptr() if d_logits is not None else None,
                                                   _stream()))

    def decode_step_async_noalloc(self, d_token, pos: int, d_next, d_logits=None) -> None:
        """mk_decode_step_async_noalloc: the step with the library's static
        scratch array in place of the bound scratch buffer."""
        self._check(self.lib.mk_decode_step_async_noalloc(self.h, d_token.data_ptr(), int(pos), d_next.data_ptr(),
                                                          d_logits.data_ptr() if d_logits is not None else None,
                                                          _stream()))

    def check_device_error(self) -> None:
        self._check(self.lib.mk_check_device_error(self.h, _stream()))

    def trace(self) -> np.ndarray:
        n = ctypes.c_size_t(0)
        self.lib.mk_get_trace(self.h, None, 0, ctypes.byref(n))  # reports the record count
        out = np.zeros(n.value, TRACE_DTYPE)
        if n.value:
            self._check(self.lib.mk_get_trace(self.h, out.ctypes.data, n.value, ctypes.byref(n)))
        return out

    def close(self):
        """Destroy the handle and release the device buffers, after the work
        queued on them has finished.  Every script calls this itself: left
        to garbage collection at interpreter exit, the buffers would be freed
        while the HIP runtime (and a profiler's hooks on it) shut down."""
        if getattr(self, "h", None):
            import torch
            torch.cuda.synchronize()
            self.lib.mk_destroy(self.h)
            self.h = None
            for name in ("weights", "kv", "rope", "scratch", "trace_buf"):
                setattr(self, name, None)
            torch.cuda.empty_cache()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _tensor_format(wfmt: int, name: str) -> str:
    if wfmt == BF16:
        return "bf16"
    if wfmt == FP8_ROW:
        return "fp8"
    return "fp8" if name in ("down", "embed") else "fp4"


def decode_codes(codec: int, d_codes, d_out) -> None:
    """Decode codes with the kernel's register decoders (0: E4M3, 1: E2M1;
    2, 3: the same through the GEMV converters; 4: fp32 values rounded to
    bf16 the way the kernel packs activations)."""
    L = load()
    rc = L.mk_decode_codes(codec, d_codes.data_ptr(), d_codes.numel(), d_out.data_ptr(), _stream())
    if rc < 0:
        raise MkError(rc, L.mk_status_str(rc).decode())


def round_bf16(d_in, d_out) -> None:
    """Round fp32 device values to bf16 the way the decode kernel packs
    activations (codec hook 4), widened back to fp32 in `d_out`."""
    L = load()
    rc = L.mk_decode_codes(4, d_in.data_ptr(), d_in.numel(), d_out.data_ptr(), _stream())
    if rc < 0:
        raise MkError(rc, L.mk_status_str(rc).decode())


def master_to_device(master, device="cuda") -> List:
    """The bf16 master (uint16 bit patterns) as torch bf16 device tensors in
    mk_pack_weights order."""
    import torch

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    order = [t(master.embed)]
    for layer in master.layers:
        for name in ("in_norm", "q", "k", "v", "q_norm", "k_norm", "o", "post_norm", "gate", "up", "down"):
            order.append(t(layer[name]))
    order.append(t(master.final_norm))
    return order
