/*
 * mk — batch-1 greedy decode of a Qwen3-style decoder as one persistent HIP
 * kernel per token on AMD MI355X (gfx950).
 *
 * What is computed follows the monolith project page
 * (projects.dotslasha.me/p/monolith): "Upstream facts" gives the model
 * (pre-norm decoder with RMSNorm, QK-norm, RoPE, grouped-query attention over
 * a KV cache, SwiGLU MLP, tied embedding used as the LM head) and the greedy
 * decode step; "Design decisions" gives the weight formats (FP8 E4M3 with one
 * scale per output row; NVFP4 = E2M1 values with one E4M3 scale per 16
 * weights and one fp32 scale per tensor; activations bf16, fp32
 * accumulation), the bf16 KV cache, the folded LM head + argmax so that one
 * launch yields one token, and the per-block phase timestamps ("X-ray").
 *
 * Conventions for every call:
 *   - Return value: MK_OK (0) or a negative mk_status.  Calls that return a
 *     token return it (>= 0) or a negative mk_status.  No exception or abort
 *     crosses this boundary.
 *   - Arguments are validated before any HIP call, so argument errors are
 *     reported the same way with or without a GPU.
 *   - The library allocates no device memory: the caller allocates the
 *     buffers whose sizes mk_query_sizes reports and binds them with mk_bind.
 *     Device pointers must be 256-byte aligned.
 *   - All work is enqueued on the caller's stream.  One model handle must not
 *     be used from two threads at once, and two launches on one handle must
 *     not run concurrently (they share the bound scratch buffer).
 *   - Matrices are [out, in] row-major (the PyTorch Linear layout).
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* mk_stream_t;  /* a hipStream_t; NULL = the null stream */

enum mk_status {
  MK_OK = 0,
  MK_E_INVALID = -1,      /* bad argument (null, out of range, misaligned) */
  MK_E_UNSUPPORTED = -2,  /* shape or format the kernels do not handle */
  MK_E_STATE = -3,        /* call out of order (e.g. decode before pack) */
  MK_E_HIP = -4,          /* a HIP runtime call failed; see mk_last_error */
  MK_E_TIMEOUT = -5,      /* a kernel wait exceeded its spin bound and the kernel exited */
};

/* Weight formats (monolith page, "Design decisions"). */
enum mk_wfmt {
  MK_WFMT_BF16 = 0,     /* every matrix bf16 */
  MK_WFMT_FP8_ROW = 1,  /* every linear and the tied embedding: E4M3, fp32 scale per row */
  MK_WFMT_FP4_MIX = 2,  /* q, k, v, o, gate, up: NVFP4; down and the tied embedding: FP8_ROW */
};

/* Model shape.  Constraints checked by mk_create: all sizes > 0;
 * n_q_heads % n_kv_heads == 0; the kernels are compiled per shape class
 * (head_dim, n_q_heads / n_kv_heads, ceil(hidden/1024),
 * ceil(n_q_heads*head_dim/1024), ceil(intermediate/1024)), one of
 * (64, 2, 1, 1, 1) and (128, 2, 1, 2, 3) (the latter is the Qwen3-0.6B shape);
 * hidden a multiple of 128; intermediate and n_q_heads*head_dim multiples
 * of 16; n_layers <= 170; max_ctx <= 1<<20.  mk_bind further needs a grid
 * with more workgroups than KV heads whose work table fits the kernel's
 * per-wave limits (the default grid, one workgroup per compute unit of an
 * MI355X, does). */
typedef struct mk_config {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab, max_ctx;
  float rope_theta;   /* RoPE base (Qwen3: 1e6) */
  float rms_eps;      /* RMSNorm epsilon (Qwen3: 1e-6) */
  int32_t wfmt;       /* mk_wfmt */
} mk_config;

/* Byte sizes of the caller-owned device buffers, plus figures used for
 * measurement. */
typedef struct mk_sizes {
  size_t weights;     /* packed weight arena (and the work table mk_bind writes after it) */
  size_t kv;          /* KV cache: n_layers * 2 * n_kv_heads * ctx4 * head_dim * 2 (bf16),
                         ctx4 = max_ctx rounded up to a multiple of 4.  Per layer l, K then V
                         (kv = 0, 1), per KV head g, a plane of ctx4 * head_dim values at element
                         ((l*2 + kv) * n_kv_heads + g) * ctx4 * head_dim.  A K plane is row-major
                         (position j, dim e at j*head_dim + e).  A V plane is tiled by 4 positions
                         (j, e at (j/4*head_dim + e)*4 + j%4), the layout the matrix-core value
                         product reads. */
  size_t rope;        /* RoPE table: max_ctx * head_dim/2 * 2 * 4 (fp32 cos, sin) */
  size_t scratch;     /* exchange buffers, argmax slots, error word, and the
                         batched prefill's buffers for 4096-position chunks
                         (residual, q/k/v outputs, GEMM input, SwiGLU output:
                         about 126 MB at the 0.6B shape) */
  size_t trace;       /* X-ray records for one step (0 in builds without X-ray) */
  size_t weight_bytes_per_token;  /* algorithmic weight bytes one step reads: every matrix,
                                     its scales and the norm gains, each once */
  size_t kv_bytes_per_position;   /* KV bytes one step reads per cached position */
} mk_sizes;

/* One X-ray record: one workgroup, one phase of one step.  Every time is an
 * s_memrealtime tick (a 100 MHz counter common to all XCDs).  Phases: 1
 * embedding; 2+6l+{0..5} layer l QKV, attention, (unused), O, gate/up, down;
 * 2+6L final norm + LM head; 3+6L argmax reduce.  A phase's input is
 * gathered by the workgroup's courier wave: t_start (gather began), t_ready
 * (every word present), t_handoff (input in LDS for the compute waves).  The
 * compute waves record t_seen (the first of them past its wait) and t_done
 * (the last of them done with its outputs).  t_mark: attention [0] scores and
 * outputs of every wave done, [1] outputs published. */
typedef struct mk_trace_rec {
  uint32_t phase;      /* phase id (above) */
  uint32_t wg;         /* workgroup index */
  uint32_t hw_id;      /* HW_ID register (CU, SE, SIMD, wave slot) */
  uint32_t xcc;        /* XCC_ID register (which XCD) */
  uint32_t active;     /* 1 if this workgroup had work in the phase */
  uint32_t pad;
  uint64_t t_start, t_ready, t_handoff, t_seen, t_done;
  uint64_t t_mark[3];
} mk_trace_rec;

typedef struct mk_model mk_model;

/* Validate `cfg` and create a host-side handle (no HIP calls).  The shape
 * is the model the monolith page decodes (Part 2, "Upstream facts": hidden
 * 1024, intermediate 3072, 28 layers, 16 query and 8 KV heads of 128, vocab
 * 151,936, tied embeddings, QK-norm, RoPE); the formats are its "Design
 * decisions" (FP8 format, NVFP4 format).  The device used is the one current
 * at mk_bind.  Errors: MK_E_INVALID (null or
 * non-positive sizes), MK_E_UNSUPPORTED (shape outside the constraints). */
int mk_create(const mk_config* cfg, mk_model** out);

/* Fill `out` with the buffer sizes for this model, and the algorithmic
 * bytes per token of the page's byte budget (Part 2, "Upstream facts":
 * weights read per step, 1,192.1 MB at bf16, and the byte-budget block that
 * follows it; its FP8 and NVFP4 lines are estimates).  No HIP calls. */
int mk_query_sizes(const mk_model* m, mk_sizes* out);

/* Register caller-owned device buffers (for example torch tensors' data
 * pointers) of at least the sizes mk_query_sizes reports; `d_trace` may be
 * NULL.  The library allocates nothing itself (the TSCT super-kernel note,
 * section 4, "Interface discipline": no workspace allocated inside an op, no
 * custom allocators).  Queries the current device's compute-unit count and sets the
 * launch grid to one workgroup per compute unit.  The pointers are not
 * owned and must stay valid until mk_destroy.  The scratch buffer and the
 * KV cache are cleared on `s`.  Errors: MK_E_INVALID (null or not 256-byte aligned),
 * MK_E_HIP (no device). */
int mk_bind(mk_model* m, void* d_weights, void* d_kv, void* d_rope, void* d_scratch,
            void* d_trace, mk_stream_t s);

/* Quantize and pack the bf16 master weights into the bound arena and build
 * the RoPE table, on the GPU (monolith page, Part 2, "Design decisions": FP8
 * format, NVFP4 format with the per-block MSE scale search, and weight layout,
 * packed in the order the kernel streams it; milestones M3 and M5, the
 * packers).  The bf16 master is taken as device tensors, not host ones: the
 * master already lives in device memory where the caller made it, and
 * quantizing there needs no device allocation inside the library (packing
 * from host memory would need a staging buffer of the library's own).  `d_tensors` holds 2 + 11*n_layers DEVICE
 * pointers to bf16 tensors in this order: embed [V,H]; per layer in_norm [H],
 * q [nq*hd,H], k [nkv*hd,H], v [nkv*hd,H], q_norm [hd], k_norm [hd],
 * o [H,nq*hd], post_norm [H], gate [I,H], up [I,H], down [H,I]; final_norm
 * [H].  Quantization follows the page's formats: FP8 per-row scale
 * s = absmax/448 and codes e4m3(w/s); NVFP4 tensor scale ts = absmax/2688,
 * block scale bs = e4m3(blockmax/(6*ts)) and codes e2m1(w/(e4m3(bs)*ts)); all
 * encodes round to nearest even and saturate.  With option 9 = k > 0 each
 * NVFP4 block's scale code is instead the one within +-k of that bs (and in
 * 0..0x7E) whose block squared error sum_i (w_i - w_hat_i)^2 is least, the
 * error summed in float64 in element order, the smaller code on a tie (the
 * page's per-block MSE scale search).  The tensors are read during
 * the call only.  Errors: MK_E_INVALID, MK_E_STATE (not bound), MK_E_HIP. */
int mk_pack_weights(mk_model* m, const void* const* d_tensors, int32_t n_tensors, mk_stream_t s);

/* Test hook for the correctness gate (monolith page, Part 2, "Hard
 * constraints": no speed number counts unless that build passed the
 * correctness suite): copy one matrix back in canonical (row-major,
 * un-fused) form, so its bytes can be compared with an independent quantizer
 * whatever the streaming layout.
 * matrix: 0 q, 1 k, 2 v, 3 o, 4 gate, 5 up, 6 down, 7 embed (layer ignored).
 * h_codes: bf16 [N,K] (uint16), FP8 [N,K] bytes, or FP4 [N,K/2] bytes (element
 * 2j in the low nibble of byte j).  h_scales: FP8 fp32 [N] (else unused).
 * h_block_scales: FP4 e4m3 [N,K/16] (else unused).  h_tensor_scale: FP4 fp32
 * (else unused).  Synchronous.  Errors: MK_E_INVALID, MK_E_STATE, MK_E_HIP. */
int mk_read_packed(mk_model* m, int32_t layer, int32_t matrix, void* h_codes, void* h_scales,
                   void* h_block_scales, float* h_tensor_scale);

/* Run the prompt through positions 0..n-1, writing the KV cache; return the
 * greedy token that follows the prompt (>= 0), or a negative mk_status
 * (monolith page, Part 2, "Design decisions", benchmark protocol: prefill
 * excluded from the timed decode).
 * By default one decode step per position; with option 10 = 1 the batched
 * prefill (chunks of positions, projections on the matrix cores).  The
 * monolith page's benchmark protocol ("Design decisions") times decode with
 * prefill excluded, so either path serves it.  Synchronous. */
int32_t mk_prefill(mk_model* m, const int32_t* h_tokens, int32_t n, mk_stream_t s);

/* One decode step (monolith page, Part 2, "Mission": the decode
 * megakernel; "Design decisions", sync experiment 5: the LM head and argmax
 * folded in, so one launch yields each token): consume `token` at position
 * `pos` (writing its K/V into the cache), attend over positions 0..pos and
 * return the next greedy token
 * (>= 0) or a negative mk_status (MK_E_INVALID if pos >= max_ctx or token is
 * outside the vocabulary; MK_E_TIMEOUT if the kernel hit its spin bound).
 * One kernel launch; synchronous (a 4-byte readback). */
int32_t mk_decode_step(mk_model* m, int32_t token, int32_t pos, mk_stream_t s);

/* The same step without any host synchronisation (monolith page, Part 2,
 * "Hard constraints": the timing harness times with events around the full
 * decode loop, outside the kernel): the token is read from device memory
 * `d_token` and the next token is written to `d_next` (both int32, device),
 * so steps chain on the device.  `d_logits` (fp32 [vocab],
 * device) receives the logits when non-NULL.  A token outside the
 * vocabulary read from `d_token` makes the kernel record MK_E_INVALID in the
 * device error word, which the next synchronous call reports.  Errors
 * (immediate): MK_E_INVALID, MK_E_STATE, MK_E_HIP. */
int mk_decode_step_async(mk_model* m, const int32_t* d_token, int32_t pos, int32_t* d_next,
                         float* d_logits, mk_stream_t s);

/* `n` greedy decode steps in one call (monolith page, Part 2, "Mission":
 * one persistent kernel per token, and the greedy loop of its benchmark):
 * the token read from `d_token` (int32, device) enters at position `pos`,
 * and step i's greedy token, the input of position pos + i + 1, is written to
 * d_next[i] (int32[n], device).  The same kernels run the steps inside as
 * few launches as possible: a launch runs several steps, every workgroup
 * reducing each step's argmax itself so that the next step starts without a
 * kernel boundary; a position with split-attention helpers (from option 8's
 * position on, when option 7 is set) runs in a launch of its own, since a
 * helper reads KV rows that another CU wrote, and a new launch also begins
 * every 512 steps and where the exchange tags would wrap.  Each step's results
 * equal those of mk_decode_step_async chained on its own tokens.
 * `d_logits` (fp32 [n][vocab], device) receives every step's logits when
 * non-NULL.  A token outside the vocabulary read from `d_token` makes the
 * kernel record MK_E_INVALID in the device error word and write -1 to
 * every d_next[i] of that launch; so does a step that hits the spin bound
 * (MK_E_TIMEOUT), for its own and the launch's later steps.  Errors
 * (immediate): MK_E_INVALID (n < 1, pos + n > max_ctx, d_token inside
 * d_next[0..n), a null buffer), MK_E_STATE, MK_E_HIP. */
int mk_decode_steps_async(mk_model* m, const int32_t* d_token, int32_t pos, int32_t n, int32_t* d_next,
                          float* d_logits, mk_stream_t s);

/* The same step as mk_decode_step_async, for callers that cannot allocate
 * device memory around it (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): its scratch (exchange words,
 * argmax words, error word, kernel parameters) is a static
 * device array of the library, 32 MiB on each GPU, held until the process
 * ends, instead of the bound scratch buffer.  The model must be bound and
 * packed (its weights, KV cache and RoPE table are used as usual); the
 * caller passes the token buffers and the optional logits as for
 * mk_decode_step_async.  The call allocates nothing: no hipMalloc, hipFree or
 * allocating library routine; it enqueues a one-word clear of the array's
 * error word, and the first call on a device, or the first after another
 * model used the array, also copies the model's parameters into it (the
 * work table lives in the weight arena, written by mk_bind).  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (two streams, two threads, two models) race and must be
 * serialised by the caller.  A failed step leaves -1 in d_next; its error
 * code is not kept.  Errors (immediate): MK_E_INVALID (as for
 * mk_decode_step_async, or another device current than the model's),
 * MK_E_STATE, MK_E_UNSUPPORTED (the model's step needs more than the array
 * holds: the size is in mk_last_error), MK_E_HIP. */
int mk_decode_step_async_noalloc(mk_model* m, const int32_t* d_token, int32_t pos, int32_t* d_next,
                                 float* d_logits, mk_stream_t s);

/* Read and clear the device error word (synchronous).  Returns MK_OK or the
 * first error a kernel recorded.  (The pages prescribe no failure handling
 * inside the kernel; every wait here is bounded instead of spinning forever,
 * and this call reports a wait that hit its bound.) */
int mk_check_device_error(mk_model* m, mk_stream_t s);

/* Copy the X-ray records of the most recent step (X-ray builds only;
 * monolith page, Part 2, "Design decisions", timing: one stamp pair per
 * block and phase in a preallocated device buffer; milestone M2: the
 * host-side dump of the trace for one chosen token position).
 * Writes min(cap, available) records; *n_out receives the number available
 * (0 in builds without X-ray).  Synchronous.  Errors: MK_E_INVALID if cap is
 * smaller than the number available. */
int mk_get_trace(mk_model* m, mk_trace_rec* h_out, size_t cap, size_t* n_out);

/* Test hook for the correctness gate (monolith page, Part 2, "Hard
 * constraints"): copy back one activation vector of the last decode step, as
 * one phase handed it to the next (the step's per-layer intermediates, for
 * op-by-op parity).  vec: 0 the q, k and v GEMV outputs before the q/k norms
 * ((nq + 2*nkv)*hd floats: the q heads, then the k heads, then the v heads);
 * 1 the attention output ((nq*hd), bf16 values, q-head order); 2 the residual
 * stream after the O-projection (hidden); 3 the SwiGLU output silu(gate)*up
 * (intermediate, bf16 values); 4 the residual stream after the down
 * projection (hidden).  `h_out` is host memory for exactly `n` floats, and n
 * must be the vector's length.  Every word must carry the last step's tag
 * (MK_E_STATE if no step ran, or a word was not written by it).  Waits for
 * the device.  Errors: MK_E_INVALID, MK_E_STATE, MK_E_HIP. */
int mk_read_exchange(mk_model* m, int32_t layer, int32_t vec, float* h_out, size_t n);

/* Test hook (monolith page, Part 2, milestone M0: run the e4m3 and e2m1
 * converts against a CPU reference for every input value): decode `n` codes
 * with the kernel's own register decoders.
 * codec 0: E4M3 bytes -> fp32; codec 1: E2M1 (one code per byte, low
 * nibble) -> fp32; codecs 2 and 3: the same two formats through the
 * converters the GEMVs use (to packed bf16), widened to fp32; codec 4:
 * `d_codes` holds n fp32 values, rounded to bf16 the way the kernel packs
 * activations and widened back.  Device buffers; enqueued on `s`.  Needs no
 * model. */
int mk_decode_codes(int32_t codec, const uint8_t* d_codes, int32_t n, float* d_out, mk_stream_t s);

/* Tuning knobs (defaults in brackets): key 0 grid size [compute units],
 * set before mk_bind (monolith page, Part 2, "Design decisions", sync
 * experiment 3: the launch-shape sweep); key 3 spin bound in 100 MHz ticks [100000000 = 1 s];
 * key 4 test hook [0]: a non-zero value shifts every tag the kernel waits
 * for, so no wait can be satisfied and each one ends at the spin bound (used
 * to test the MK_E_TIMEOUT path without hanging); key 5 poll back-off
 * between exchange poll rounds, 0..16 units of about 512 clocks [0]; key 6
 * launch mode [-1]: 0 launches each step cooperatively (the runtime checks
 * that the grid is resident at once; on MI355X this adds about 20 us between
 * consecutive steps), 1 with a plain launch, allowed only when mk_bind found
 * that the device holds the whole grid at once, -1 plain when it does, else
 * cooperative.  The kernel's waits assume that every workgroup runs: should
 * another process hold compute units during a plain launch, they end at the
 * spin bound with MK_E_TIMEOUT instead of hanging.  Keys 7 and 8, split
 * attention [192, 704]: with key 7 = c > 0, a step at a position pos at or
 * past key 8 spreads KV head g's cached positions over its home workgroup and
 * ns = min(helpers, pos / c) helper workgroups on the same XCD (helpers = the
 * GEMV workgroups there, at most 32 per head), each taking an equal slice;
 * the home merges their partial (maximum, sum, output) triples with the
 * log-sum-exp rule.  c = 0 turns it off.  (On MI355X at the 0.6B shape the
 * split path is faster from about 700 cached positions on, where consecutive
 * positions run one launch each; below, the home alone within one launch of
 * several steps is faster.)  Key 9, NVFP4
 * block scale search radius 0..126 [0], set before mk_pack_weights (see
 * there); 0 keeps the absolute-maximum recipe.  Key 10, prefill path [0]:
 * 0 runs mk_prefill as one decode launch per prompt position; 1 runs the
 * prompt through each layer in chunks of 4096 positions, the projections as
 * matrix products on the matrix cores (bf16 operands, fp32 accumulation,
 * weights dequantized exactly), with the decode path's rounding points; it
 * writes the same KV cache up to summation order.  1 needs hidden,
 * intermediate and n_q_heads*head_dim divisible by 64, hidden <= 4096 and
 * head_dim 64 or 128 (else MK_E_UNSUPPORTED).
 * Key 11, synchronisation between phases [0]: 0 tagged exchange words (each
 * consumer waits for exactly the values it reads); 1 and 2 one grid-wide
 * barrier per phase hand-off, the monolith page's baseline kept for
 * comparison ("Upstream facts": four full-grid atomic barriers per layer;
 * "Design decisions": the sync experiments measure the counters against
 * them): every workgroup arrives at an agent-scope counter once its stores
 * of the phase are complete, and every consumer waits for the last arrival
 * before reading.  Mode 1 uses relaxed counter atomics (the values travel in
 * device-coherent words); mode 2 arrives with an agent-scope release and
 * leaves with an agent-scope acquire, the literal reading of the page's
 * release/acquire counters (on MI355X an L2 write-back and an L2 invalidate
 * of the workgroup's XCD at every barrier).  Modes 1 and 2 turn split
 * attention off and are refused by mk_decode_step_async_noalloc.
 * Key 12, LM-head balancing [0], for launches of several steps
 * (mk_decode_steps_async): 1 moves each workgroup's share of the LM-head rows
 * towards equal end times, from the step before's timings (a damped step;
 * which workgroup computes a row changes no result); 0 keeps equal shares.
 * On MI355X the balancing measured slower than equal shares (the per-XCD
 * LM-head speed does not persist from one step to the next), hence off.
 * Keys 1 and 2 are reserved.
 * Errors: MK_E_INVALID (unknown key, value out of range), MK_E_STATE. */
int mk_set_option(mk_model* m, int32_t key, int64_t value);

/* 1 if the library was built with the X-ray stamps, else 0 (monolith page,
 * Part 2, "Hard constraints": X-ray compiles only behind a compile-time flag,
 * and headline numbers come only from uninstrumented builds). */
int mk_has_xray(void);

/* Diagnostics: the text of a status code; the last error message of a handle
 * (owned by the handle, valid until its next call). */
const char* mk_status_str(int status);
const char* mk_last_error(const mk_model* m);
/* Free the host handle.  The caller's device buffers are not touched. */
void mk_destroy(mk_model* m);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
