// gfx950 kernels that run once per model: the weight packers (the page's
// FP8 and NVFP4 recipes), the RoPE table builder, and a codec test hook.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <stdint.h>

#include "mk_codec.h"
#include "mk_launch.h"

namespace mk {

__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// ---------------------------------------------------------------- packing
// bf16 rows copied into place.  dst row of source row r: row_off + r*row_step.
__global__ void pack_bf16_kernel(const uint16_t* src, int N, int K, uint16_t* dst, int row_off, int row_step) {
  const int r = blockIdx.x;
  if (r >= N) return;
  const uint16_t* s = src + (size_t)r * K;
  uint16_t* d = dst + (size_t)(row_off + (size_t)r * row_step) * K;
  for (int k = threadIdx.x; k < K; k += blockDim.x) d[k] = s[k];
}

__device__ __forceinline__ float block_max_256(float v, float* red) {
  v = wave_max64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

// FP8 per output row: s = absmax/448 (1 for a zero row), c = e4m3(w/s).
__global__ void pack_fp8_kernel(const uint16_t* src, int N, int K, uint8_t* codes, float* scales, int row_off,
                                int row_step) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  if (r >= N) return;
  const uint16_t* s = src + (size_t)r * K;
  float a = 0.f;
  for (int k = threadIdx.x; k < K; k += blockDim.x) a = fmaxf(a, fabsf(bf16_to_f32(s[k])));
  a = block_max_256(a, red);
  const float sc = a == 0.f ? 1.0f : a / 448.0f;
  const size_t dr = row_off + (size_t)r * row_step;
  for (int k = threadIdx.x; k < K; k += blockDim.x) codes[dr * K + k] = (uint8_t)f32_to_e4m3(bf16_to_f32(s[k]) / sc);
  if (threadIdx.x == 0) scales[dr] = sc;
}

// Absolute maximum of a whole tensor (non-negative floats order like their bits).
__global__ void amax_kernel(const uint16_t* src, size_t n, uint32_t* out) {
  __shared__ float red[16];
  float a = 0.f;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    a = fmaxf(a, fabsf(bf16_to_f32(src[i])));
  a = block_max_256(a, red);
  if (threadIdx.x == 0) atomicMax(out, __float_as_uint(a));
}

// One E2M1 code's value (sign bit 3; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const float m = (c & 4u) ? (float)(2u + (c & 1u)) * (float)(1u << ((c >> 1) & 1u)) : 0.5f * (float)(c & 3u);
  return (c & 8u) ? -m : m;
}

// Squared error of one 16-wide block stored with effective scale eff:
// sum_i (w_i - fl32(e2m1(c_i) * eff))^2 with c_i = e2m1(fl32(w_i / eff)),
// every code 0 when eff = 0.  Differences, squares and the running sum are
// float64 operations in index order, each rounded on its own.
__device__ double fp4_block_sq_error(const float* w, float eff) {
  double e = 0.0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float q = eff != 0.f ? __fmul_rn(e2m1_value(f32_to_e2m1(w[k] / eff)), eff) : 0.f;
    const double d = __dsub_rn((double)w[k], (double)q);
    e = __dadd_rn(e, __dmul_rn(d, d));
  }
  return e;
}

// NVFP4: ts = A/2688 (1 if A = 0); per 16-block the absolute-maximum scale
// code b0 = e4m3(a_b/fl32(6 ts)); with search > 0 the block scale is the code
// in [b0 - search, b0 + search] (within 0..0x7E) of least block squared error,
// the smaller code on a tie (the MSE scale search of the page's NVFP4 format);
// eff = e4m3(bs) * ts, c = e2m1(w/eff) (all 0 when eff = 0).  One thread per block.
__global__ void pack_fp4_kernel(const uint16_t* src, int N, int K, uint8_t* codes, uint8_t* bscales, float* tscale,
                                int ts_index, const uint32_t* amax, int row_off, int row_step, int search) {
  const int r = blockIdx.x;
  if (r >= N) return;
  const float A = __uint_as_float(*amax);
  const float ts = A == 0.f ? 1.0f : A / 2688.0f;
  if (r == 0 && threadIdx.x == 0) tscale[ts_index] = ts;
  const float six_ts = 6.0f * ts;
  const size_t dr = row_off + (size_t)r * row_step;
  for (int b = threadIdx.x; b < K / 16; b += blockDim.x) {
    const uint16_t* s = src + (size_t)r * K + b * 16;
    float w[16];
    float ab = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      w[k] = bf16_to_f32(s[k]);
      ab = fmaxf(ab, fabsf(w[k]));
    }
    uint32_t bs = f32_to_e4m3(ab / six_ts);
    if (search > 0) {
      const int lo = max((int)bs - search, 0), hi = min((int)bs + search, 0x7E);
      double best = 0.0;
      for (int c = lo; c <= hi; ++c) {   // ascending: a tie keeps the smaller code
        const double e = fp4_block_sq_error(w, __fmul_rn(e4m3_to_f32((uint32_t)c), ts));
        if (c == lo || e < best) {
          best = e;
          bs = (uint32_t)c;
        }
      }
    }
    const float eff = __fmul_rn(e4m3_to_f32(bs), ts);
    uint32_t lo = 0, hi = 0;
    if (eff != 0.f) {
#pragma unroll
      for (int k = 0; k < 8; ++k) lo |= f32_to_e2m1(w[k] / eff) << (4 * k);
#pragma unroll
      for (int k = 0; k < 8; ++k) hi |= f32_to_e2m1(w[8 + k] / eff) << (4 * k);
    }
    uint32_t* c = reinterpret_cast<uint32_t*>(codes + dr * (K / 2) + b * 8);
    c[0] = lo;
    c[1] = hi;
    bscales[dr * (K / 16) + b] = (uint8_t)bs;
  }
}

// RoPE table: cos and sin of p * theta^(-2i/hd), angle in double, rounded to float.
__global__ void rope_kernel(float* out, int max_ctx, int hd, double theta) {
  const size_t n = (size_t)max_ctx * (hd / 2);
  for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < n; t += (size_t)gridDim.x * blockDim.x) {
    const int p = (int)(t / (hd / 2)), i = (int)(t % (hd / 2));
    const double omega = pow(theta, (-2.0 * (double)i) / (double)hd);
    const double ang = (double)p * omega;
    out[2 * t] = (float)cos(ang);
    out[2 * t + 1] = (float)sin(ang);
  }
}

__global__ void decode_codes_kernel(int codec, const uint8_t* in, int n, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t b = in[i];
  if (codec == 0) {
    out[i] = e4m3_to_f32(b);
  } else if (codec == 1) {
    float f[8];
    e2m1x8_to_f32(b & 0xFu, f);
    out[i] = f[0];
  } else if (codec == 2) {   // E4M3 -> bf16 converter (the GEMV path), byte in position 2
    out[i] = bf16_lo(e4m3x2_to_bf16x2<true>(b << 16));
  } else {                   // E2M1 -> bf16 converter (the GEMV path), nibble in the high half of byte 1
    out[i] = bf16_hi(e2m1x2_to_bf16x2<1>((b & 0xFu) << 12));
  }
}

// fp32 -> bf16 as the decode kernel packs activations (pairs), widened back.
__global__ void round_bf16_kernel(const float* in, int n, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (2 * i >= n) return;
  const float a = in[2 * i], b = 2 * i + 1 < n ? in[2 * i + 1] : 0.f;
  const uint32_t w = pack_bf16(a, b);
  out[2 * i] = bf16_lo(w);
  if (2 * i + 1 < n) out[2 * i + 1] = bf16_hi(w);
}

// ------------------------------------------------------- launch wrappers
__global__ void zero_words_kernel(uint64_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

hipError_t launch_zero_words(uint64_t* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>(1024, (n + 255) / 256);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_pack_bf16(const uint16_t* src, int N, int K, uint16_t* dst, int row_off, int row_step,
                            hipStream_t s) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(pack_bf16_kernel, dim3(N), dim3(256), 0, s, src, N, K, dst, row_off, row_step);
  return hipGetLastError();
}

hipError_t launch_pack_fp8(const uint16_t* src, int N, int K, uint8_t* codes, float* scales, int row_off,
                           int row_step, hipStream_t s) {
  hipLaunchKernelGGL(pack_fp8_kernel, dim3(N), dim3(256), 0, s, src, N, K, codes, scales, row_off, row_step);
  return hipGetLastError();
}

hipError_t launch_pack_fp4(const uint16_t* src, int N, int K, uint8_t* codes, uint8_t* bscales, float* tscale,
                           int ts_index, uint32_t* amax, int row_off, int row_step, int search, hipStream_t s) {
  hipError_t e = hipMemsetAsync(amax, 0, 4, s);
  if (e != hipSuccess) return e;
  const size_t n = (size_t)N * K;
  hipLaunchKernelGGL(amax_kernel, dim3(1024), dim3(256), 0, s, src, n, amax);
  hipLaunchKernelGGL(pack_fp4_kernel, dim3(N), dim3(64), 0, s, src, N, K, codes, bscales, tscale, ts_index, amax,
                     row_off, row_step, search);
  return hipGetLastError();
}

hipError_t launch_rope(float* out, int max_ctx, int hd, double theta, hipStream_t s) {
  hipLaunchKernelGGL(rope_kernel, dim3(1024), dim3(256), 0, s, out, max_ctx, hd, theta);
  return hipGetLastError();
}

hipError_t launch_decode_codes(int codec, const uint8_t* in, int n, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (codec == 4) {
    hipLaunchKernelGGL(round_bf16_kernel, dim3((n / 2 + 256) / 256), dim3(256), 0, s,
                       reinterpret_cast<const float*>(in), n, out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(decode_codes_kernel, dim3((n + 255) / 256), dim3(256), 0, s, codec, in, n, out);
  return hipGetLastError();
}

}  // namespace mk
