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
// `ns` > 0 launches the split-attention variant with ns helpers per KV head.
hipError_t launch_decode(const Params* d_params, int wfmt, int hd, int gs, int hidden, int qdim, int inter, int grid,
                         bool cooperative, const int32_t* d_token, int pos, int ns, uint32_t epoch, int32_t* d_next,
                         float* d_logits, hipStream_t s);
// Workgroups of the decode kernel (either variant) that one compute unit holds at once.
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
}  // namespace mk
