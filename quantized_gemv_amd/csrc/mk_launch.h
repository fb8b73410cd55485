// Host-side entry points into the kernel sources (used by the C-ABI layer).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_shared.h"

namespace mk {
// `d_params` points to a Params copy in device memory that stays unchanged while the kernel runs.
// `cooperative`: hipLaunchCooperativeKernel (the runtime guarantees that the
// whole grid is resident) or a plain launch (the caller has checked with
// decode_coresident() that the grid fits the device at once).
// `ns` > 0 launches the split-attention variant with ns helpers per KV head;
// `barrier` the grid-barrier variant (needs ns == 0).
hipError_t launch_decode(const Params* d_params, int wfmt, int hd, int gs, int hidden, int qdim, int inter, int grid,
                         bool cooperative, bool barrier, const int32_t* d_token, int pos, int nsteps, int ns,
                         uint32_t epoch, int32_t* d_next, float* d_logits, hipStream_t s);
// Workgroups of the decode kernel (any variant) that one compute unit holds at once.
hipError_t decode_coresident(int wfmt, int hd, int gs, int hidden, int qdim, int inter, int* per_cu);
bool decode_shape_supported(int hd, int gs, int hidden, int qdim, int inter);
hipError_t launch_pack_bf16(const uint16_t* src, int N, int K, uint16_t* dst, int row_off, int row_step,
                            hipStream_t s);
hipError_t launch_pack_fp8(const uint16_t* src, int N, int K, uint8_t* codes, float* scales, int row_off,
                           int row_step, hipStream_t s);
hipError_t launch_pack_fp4(const uint16_t* src, int N, int K, uint8_t* codes, uint8_t* bscales, float* tscale,
                           int ts_index, uint32_t* amax, int row_off, int row_step, int search, hipStream_t s);
hipError_t launch_rope(float* out, int max_ctx, int hd, double theta, hipStream_t s);
hipError_t launch_decode_codes(int codec, const uint8_t* in, int n, float* out, hipStream_t s);
// Set n 64-bit words to zero with a kernel (no hipMemsetAsync, so the clear
// is an ordinary kernel node when the caller captures the stream).
hipError_t launch_zero_words(uint64_t* p, size_t n, hipStream_t s);

// Batched prefill (mk_prefill.hip): positions [c0, c0 + cn) of a prompt
// through every layer; with `last`, also the LM head of position c0+cn-1 and
// its argmax into *next.  Device pointers; the workspace buffers hold
// kPrefillChunk rows.
constexpr int kPrefillChunk = 4096;
constexpr int kPrefillHeadGroups = 256;   // LM-head workgroups (4 waves each)
struct PrefillArgs {
  const Params* params;
  const Mat *mat_qkv, *mat_o, *mat_gu, *mat_down;   // inside the device Params
  uint32_t fmt_lin, fmt_down;
  uint64_t layer_stride, in_norm, post_norm;
  int L, H, hd, nq, nkv, I;
  int c0, cn;
  bool last;
  const int32_t* tokens;   // the chunk's tokens
  float *X, *QKV;          // [chunk][H], [chunk][(nq + 2 nkv) hd]
  uint16_t *A, *Hb;        // [chunk][max(H, nq hd)], [chunk][I] bf16
  float* best_v;           // [kPrefillHeadGroups * 4]
  int32_t* best_i;
  int32_t* next;
  float* logits;           // [vocab] or null
};
hipError_t launch_prefill_chunk(const PrefillArgs& a, hipStream_t s);
}  // namespace mk
