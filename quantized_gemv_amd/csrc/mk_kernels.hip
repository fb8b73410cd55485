// gfx950 kernels: the persistent batch-1 decode kernel, the weight packers
// and the RoPE table builder.
//
// One launch computes one greedy decode step of a Qwen3-style decoder (the
// model of the monolith project page, "Upstream facts"): embedding lookup,
// then per layer RMSNorm -> fused QKV GEMV -> q/k RMSNorm + RoPE + KV append
// -> GQA attention -> O-projection + residual -> RMSNorm -> gate/up GEMV +
// SwiGLU -> down GEMV + residual, then the final RMSNorm, the tied LM-head
// GEMV and the argmax, so one launch yields one token (the page's "fold the LM
// head and argmax into the megakernel").
//
// Launch: cooperative, one workgroup of 512 threads per compute unit, so all
// workgroups are resident and may wait on each other.  Each phase splits its
// rows (or attention units) over the workgroups; a workgroup issues its
// weight loads for the phase first and only then waits for the phase's input
// vector, which arrives through the tagged-word exchange of mk_sync.h.
// Weights are dequantized in registers (FP8 and FP4 through the gfx950
// converters) and every product accumulates in fp32 (the page's W8A16 scheme;
// the pages' contract also asks for each weight byte to be read once per
// token and for fp32 accumulation).  No MFMA: these are matrix-vector
// products, bound by HBM bandwidth.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mk.h"
#include "mk_codec.h"
#include "mk_shared.h"
#include "mk_sync.h"
#include "mk_xray.h"

namespace mk {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

constexpr int kMaxAct = 2048;        // bf16 pairs of a normalized input (hidden <= 4096)
constexpr int kAttBlock = kThreads;  // positions scored per attention block
constexpr int kMaxGroupDim = 512;    // (q heads per KV head) * head_dim
constexpr int kMaxGroup = 4;         // q heads per KV head
constexpr int kGemvBatch = 4;        // GEMV items per wave in flight

struct AttSmem {
  float q[kMaxGroupDim];             // normed + roped q of the group's heads
  float k[256], v[256];              // this position's k (normed, roped) and v
  uint32_t kb[128], vb[128];         // the same as bf16 pairs (what the cache holds)
  float pr[kMaxGroup][kAttBlock];    // scores, then probabilities, of one block
  float o[kWaves][kMaxGroupDim];     // per-wave partial outputs
  float m[kMaxGroup], l[kMaxGroup], sc[kMaxGroup];
};
struct GemvSmem {
  uint32_t act[kMaxAct];             // normalized input as bf16 pairs
  float part[kMaxPart];              // partial dot products per (row, 1024-chunk)
  float y[kMaxPart];                 // finished rows
};
struct Smem {
  uint32_t vin[kMaxVecWords];        // gathered payloads
  union {
    AttSmem att;
    GemvSmem g;
  } u;
  float red[kWaves * 2];
  int32_t redi[kWaves];
  float x_own[kMaxOwn];              // residual rows this workgroup owns
};

__device__ __forceinline__ Mat at_layer(const Mat& m, uint64_t off) {
  Mat r = m;
  r.codes += off;
  r.scales += off;
  r.tscale += off;
  return r;
}

__device__ __forceinline__ void split_range(int n, int parts, int i, int& a, int& b) {
  a = (int)((int64_t)n * i / parts);
  b = (int)((int64_t)n * (i + 1) / parts);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Sum over the workgroup, same value in every thread, fixed order.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += red[w];
  return s;
}

// act[j] = bf16 pair of g * (x * r) at 2j, 2j+1, with r = 1/sqrt(mean(x^2) + eps)
// (RMSNorm; every workgroup computes the factor itself, the page's trick for
// removing a barrier).
__device__ __forceinline__ void rmsnorm_to_act(const Params& p, const uint32_t* xin, uint64_t g_off, int n,
                               uint32_t* act, float* red) {
  float ss = 0.f;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const float x = __uint_as_float(xin[i]);
    ss = fmaf(x, x, ss);
  }
  const float tot = block_sum(ss, red);
  const float r = 1.0f / sqrtf(tot / (float)n + p.eps);
  const uint16_t* g = reinterpret_cast<const uint16_t*>(p.w + g_off);
  for (int j = threadIdx.x; j < n / 2; j += kThreads) {
    const float a = bf16_to_f32(g[2 * j]) * (__uint_as_float(xin[2 * j]) * r);
    const float b = bf16_to_f32(g[2 * j + 1]) * (__uint_as_float(xin[2 * j + 1]) * r);
    act[j] = f32_to_bf16(a) | (f32_to_bf16(b) << 16);
  }
}

// ------------------------------------------------------------------ GEMV
// Work item = (row, 1024-element chunk of K).  Lane l of a wave covers
// elements [c*1024 + 16 l, +16) of its item's row, so a wave streams one
// contiguous 1 KB (fp8) / 2 KB (bf16) / 512 B (fp4) run per item with
// 16-byte loads.  Items are dealt to waves round-robin; each wave keeps
// kGemvBatch items' weights in flight.
template <uint32_t FMT>
struct Batch {
  v4u w0[kGemvBatch], w1[kGemvBatch];
};

template <uint32_t FMT>
__device__ __forceinline__ void gemv_load(const Params& p, const Mat& m, int r0, int items, int nch,
                                          int bi, Batch<FMT>& B) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < kGemvBatch; ++u) {
    const int it = wave + kWaves * (bi * kGemvBatch + u);
    const int rr = it / nch, c = it - rr * nch;
    const int e0 = c * 1024 + lane * 16;
    if (it < items && e0 < (int)m.K) {
      const uint64_t row = (uint64_t)(r0 + rr);
      const uint8_t* base = p.w + m.codes;
      if (FMT == FMT_BF16) {
        const v4u* q = reinterpret_cast<const v4u*>(base + (row * m.K + e0) * 2);
        B.w0[u] = q[0];
        B.w1[u] = q[1];
      } else if (FMT == FMT_FP8) {
        B.w0[u] = *reinterpret_cast<const v4u*>(base + row * m.K + e0);
      } else {
        const v2u c2 = *reinterpret_cast<const v2u*>(base + (row * m.K + e0) / 2);
        B.w0[u].x = c2.x;
        B.w0[u].y = c2.y;
        B.w1[u].x = p.w[m.scales + row * (m.K / 16) + e0 / 16];
      }
    }
  }
}

__device__ __forceinline__ float fp4_tensor_scale(const Params& p, const Mat& m, uint32_t row) {
  uint32_t idx = 0;
  if (m.ts_mode == 1) idx = row < m.ts_b0 ? 0u : (row < m.ts_b1 ? 1u : 2u);
  else if (m.ts_mode == 2) idx = row & 1u;
  return *reinterpret_cast<const float*>(p.w + m.tscale + 4 * idx);
}

template <uint32_t FMT>
__device__ __forceinline__ void gemv_compute(const Params& p, const Mat& m, int r0, int items, int nch,
                                             int bi, const Batch<FMT>& B, const uint32_t* act,
                                             float* part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float acc[kGemvBatch];
#pragma unroll
  for (int u = 0; u < kGemvBatch; ++u) {
    const int it = wave + kWaves * (bi * kGemvBatch + u);
    const int rr = it / nch, c = it - rr * nch;
    const int e0 = c * 1024 + lane * 16;
    float a = 0.f;
    if (it < items && e0 < (int)m.K) {
      const v4u* av = reinterpret_cast<const v4u*>(act + e0 / 2);
      const v4u x0 = av[0], x1 = av[1];
      const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      if (FMT == FMT_BF16) {
        const uint32_t ws[8] = {B.w0[u].x, B.w0[u].y, B.w0[u].z, B.w0[u].w,
                                B.w1[u].x, B.w1[u].y, B.w1[u].z, B.w1[u].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          a = fmaf(bf16_lo(ws[j]), bf16_lo(xs[j]), a);
          a = fmaf(bf16_hi(ws[j]), bf16_hi(xs[j]), a);
        }
      } else if (FMT == FMT_FP8) {
        const uint32_t ws[4] = {B.w0[u].x, B.w0[u].y, B.w0[u].z, B.w0[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float f[4];
          e4m3x4_to_f32(ws[j], f);
          a = fmaf(f[0], bf16_lo(xs[2 * j]), a);
          a = fmaf(f[1], bf16_hi(xs[2 * j]), a);
          a = fmaf(f[2], bf16_lo(xs[2 * j + 1]), a);
          a = fmaf(f[3], bf16_hi(xs[2 * j + 1]), a);
        }
      } else {
        const uint32_t ws[2] = {B.w0[u].x, B.w0[u].y};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float f[8];
          e2m1x8_to_f32(ws[j], f);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            a = fmaf(f[2 * t], bf16_lo(xs[4 * j + t]), a);
            a = fmaf(f[2 * t + 1], bf16_hi(xs[4 * j + t]), a);
          }
        }
        const uint32_t row = (uint32_t)(r0 + rr);
        a *= e4m3_to_f32(B.w1[u].x) * fp4_tensor_scale(p, m, row);
      }
    }
    acc[u] = a;
  }
#pragma unroll
  for (int u = 0; u < kGemvBatch; ++u) acc[u] = wave_sum(acc[u]);
  if (lane == 0) {
#pragma unroll
    for (int u = 0; u < kGemvBatch; ++u) {
      const int it = wave + kWaves * (bi * kGemvBatch + u);
      if (it < items) part[it] = acc[u];
    }
  }
}

// Rows [r0, r0+nrows) of `m` against the bf16 vector `act`: y[t] for t < nrows.
// The first batch of weights must already be in `B`.
template <uint32_t FMT>
__device__ __forceinline__ void gemv_rows(const Params& p, const Mat& m, int r0, int nrows, Batch<FMT>& B,
                          const uint32_t* act, float* part, float* y) {
  const int nch = ((int)m.K + 1023) >> 10;
  const int items = nrows * nch;
  const int wave = threadIdx.x >> 6;
  gemv_compute<FMT>(p, m, r0, items, nch, 0, B, act, part);
  for (int bi = 1; wave + kWaves * bi * kGemvBatch < items; ++bi) {
    gemv_load<FMT>(p, m, r0, items, nch, bi, B);
    gemv_compute<FMT>(p, m, r0, items, nch, bi, B, act, part);
  }
  __syncthreads();
  for (int t = threadIdx.x; t < nrows; t += kThreads) {
    float s = 0.f;
    for (int c = 0; c < nch; ++c) s += part[t * nch + c];
    if (FMT == FMT_FP8) s *= *reinterpret_cast<const float*>(p.w + m.scales + 4ull * (uint64_t)(r0 + t));
    y[t] = s;
  }
  __syncthreads();
}

// A GEMV phase: prefetch the first batch of weights, wait for the input
// vector, optionally RMSNorm it, and compute the workgroup's rows into y.
template <uint32_t FMT>
__device__ __forceinline__ bool gemv_phase_t(const Params& p, Smem& s, const Mat& m, int r0, int nrows,
                             const uint64_t* src, int nwords, uint32_t tag, uint64_t norm_g,
                             XrayClock& xc) {
  Batch<FMT> B;
  const int nch = ((int)m.K + 1023) >> 10;
  if (nrows > 0) gemv_load<FMT>(p, m, r0, nrows * nch, nch, 0, B);
  XR_WAIT_BEGIN(xc);
  const bool ok = gather(src, nwords, tag, s.vin, p);
  if (__syncthreads_or(!ok)) return false;
  XR_WAIT_END(xc);
  if (nrows <= 0) return true;
  XR_ACTIVE(xc);
  const uint32_t* act = s.vin;
  if (norm_g) {
    rmsnorm_to_act(p, s.vin, norm_g, (int)m.K, s.u.g.act, s.red);
    __syncthreads();
    act = s.u.g.act;
  }
  gemv_rows<FMT>(p, m, r0, nrows, B, act, s.u.g.part, s.u.g.y);
  return true;
}

__device__ __forceinline__ bool gemv_phase(const Params& p, Smem& s, const Mat& m, int r0, int nrows, const uint64_t* src,
                           int nwords, uint32_t tag, uint64_t norm_g, XrayClock& xc) {
  if (m.fmt == FMT_FP8) return gemv_phase_t<FMT_FP8>(p, s, m, r0, nrows, src, nwords, tag, norm_g, xc);
  if (m.fmt == FMT_FP4) return gemv_phase_t<FMT_FP4>(p, s, m, r0, nrows, src, nwords, tag, norm_g, xc);
  return gemv_phase_t<FMT_BF16>(p, s, m, r0, nrows, src, nwords, tag, norm_g, xc);
}

// ------------------------------------------------------------- attention
// How many position splits per KV head at this context length: about
// att_target positions per unit, at most ns_max, and no empty split.
__device__ __forceinline__ void att_split(const Params& p, int n, int& ns, int& span) {
  ns = (n + p.att_target - 1) / p.att_target;
  if (ns > p.ns_max) ns = p.ns_max;
  if (ns < 1) ns = 1;
  span = (n + ns - 1) / ns;
  ns = (n + span - 1) / span;
}

// RMSNorm (gain g, head_dim hd) then RoPE at `pos` of one head vector held in
// LDS, by one wave.  Rotate-half pairs (i, i + hd/2).
__device__ __forceinline__ void head_norm_rope(const Params& p, float* v, uint64_t g_off, int pos) {
  const int lane = threadIdx.x & 63, hd = p.hd;
  float ss = 0.f;
  for (int d = lane; d < hd; d += 64) ss = fmaf(v[d], v[d], ss);
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)hd + p.eps);
  const uint16_t* g = reinterpret_cast<const uint16_t*>(p.w + g_off);
  const float* cs = p.rope + (size_t)pos * hd;  // [hd/2][2]
  const int half = hd / 2;
  for (int i = lane; i < half; i += 64) {
    const float a = bf16_to_f32(g[i]) * (v[i] * r);
    const float b = bf16_to_f32(g[i + half]) * (v[i + half] * r);
    const float c = cs[2 * i], sn = cs[2 * i + 1];
    v[i] = a * c - b * sn;
    v[i + half] = b * c + a * sn;
  }
}

// One unit = (KV head g, position split): scores of the group's q heads over
// the split's positions with an online softmax, producing either the final
// output (one split) or (max, sum, unnormalized output) for the merge.
__device__ __forceinline__ bool attention_unit(const Params& p, Smem& s, int l, int g, int sidx, int ns, int span, int pos,
                               uint32_t epoch) {
  AttSmem& A = s.u.att;
  const int hd = p.hd, gs = p.nq / p.nkv, nq = p.nq, nkv = p.nkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j0 = sidx * span, j1 = min(j0 + span, pos + 1);
  const int par = l & 1;
  const uint32_t tag_qkv = make_tag(epoch, 6 * l + 2);
  const uint64_t* qkv = p.xch + p.x.qkv + (uint64_t)par * p.x.par_qkv +
                        (uint64_t)(blockIdx.x % p.R) * p.x.rep_qkv;
  bool ok = gather(qkv + (uint64_t)g * gs * hd, gs * hd, tag_qkv, reinterpret_cast<uint32_t*>(A.q), p);
  ok = ok && gather(qkv + (uint64_t)(nq + g) * hd, hd, tag_qkv, reinterpret_cast<uint32_t*>(A.k), p);
  ok = ok && gather(qkv + (uint64_t)(nq + nkv + g) * hd, hd, tag_qkv, reinterpret_cast<uint32_t*>(A.v), p);
  if (__syncthreads_or(!ok)) return false;

  const Layer& L0 = p.layer0;
  const uint64_t loff = (uint64_t)l * p.layer_stride;
  if (wave < gs) head_norm_rope(p, A.q + wave * hd, L0.q_norm + loff, pos);
  else if (wave == gs) head_norm_rope(p, A.k, L0.k_norm + loff, pos);
  __syncthreads();
  for (int t = threadIdx.x; t < hd / 2; t += kThreads) {
    A.kb[t] = f32_to_bf16(A.k[2 * t]) | (f32_to_bf16(A.k[2 * t + 1]) << 16);
    A.vb[t] = f32_to_bf16(A.v[2 * t]) | (f32_to_bf16(A.v[2 * t + 1]) << 16);
  }
  __syncthreads();
  const size_t plane = (size_t)p.max_ctx * hd;  // bf16 elements per (layer, k|v, head)
  uint32_t* kc = reinterpret_cast<uint32_t*>(p.kv + ((size_t)(l * 2 + 0) * nkv + g) * plane);
  uint32_t* vc = reinterpret_cast<uint32_t*>(p.kv + ((size_t)(l * 2 + 1) * nkv + g) * plane);
  if (j0 <= pos && pos < j1) {
    for (int t = threadIdx.x; t < hd / 2; t += kThreads) {
      kc[(size_t)pos * (hd / 2) + t] = A.kb[t];
      vc[(size_t)pos * (hd / 2) + t] = A.vb[t];
    }
  }
  // bf16 k/v of this position, as the cache holds them
  for (int t = threadIdx.x; t < hd / 2; t += kThreads) {
    A.k[2 * t] = bf16_lo(A.kb[t]);
    A.k[2 * t + 1] = bf16_hi(A.kb[t]);
    A.v[2 * t] = bf16_lo(A.vb[t]);
    A.v[2 * t + 1] = bf16_hi(A.vb[t]);
  }
  if (threadIdx.x < kMaxGroup) {
    A.m[threadIdx.x] = -INFINITY;
    A.l[threadIdx.x] = 0.f;
  }
  const int dpl = hd / 64;  // dims per lane in the PV product (1, 2 or 4)
  float o[kMaxGroup][4];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
    for (int k = 0; k < 4; ++k) o[h][k] = 0.f;
  const float rs = sqrtf((float)hd);
  __syncthreads();

  for (int jb = j0; jb < j1; jb += kAttBlock) {
    const int nb = min(kAttBlock, j1 - jb);
    // scores: one position per thread
    if ((int)threadIdx.x < nb) {
      const int j = jb + threadIdx.x;
      float dot[kMaxGroup] = {0.f, 0.f, 0.f, 0.f};
      if (j == pos) {
        for (int d = 0; d < hd; ++d) {
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h)
            if (h < gs) dot[h] = fmaf(A.q[h * hd + d], A.k[d], dot[h]);
        }
      } else {
        const v4u* kr = reinterpret_cast<const v4u*>(kc + (size_t)j * (hd / 2));
        for (int c = 0; c < hd / 8; ++c) {
          const v4u w = kr[c];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int d = c * 8 + 2 * e;
            const float k0 = bf16_lo(ws[e]), k1 = bf16_hi(ws[e]);
#pragma unroll
            for (int h = 0; h < kMaxGroup; ++h) {
              if (h < gs) {
                dot[h] = fmaf(A.q[h * hd + d], k0, dot[h]);
                dot[h] = fmaf(A.q[h * hd + d + 1], k1, dot[h]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
        if (h < gs) A.pr[h][threadIdx.x] = dot[h] / rs;
    }
    __syncthreads();
    // block max and new running max, one wave per head
    if (wave < gs) {
      float mx = -INFINITY;
      for (int t = lane; t < nb; t += 64) mx = fmaxf(mx, A.pr[wave][t]);
      mx = wave_max(mx);
      if (lane == 0) {
        const float mn = fmaxf(A.m[wave], mx);
        A.sc[wave] = expf(A.m[wave] - mn);
        A.m[wave] = mn;
      }
    }
    __syncthreads();
    if ((int)threadIdx.x < nb)
      for (int h = 0; h < gs; ++h) A.pr[h][threadIdx.x] = expf(A.pr[h][threadIdx.x] - A.m[h]);
    __syncthreads();
    if (wave < gs) {
      float sm = 0.f;
      for (int t = lane; t < nb; t += 64) sm += A.pr[wave][t];
      sm = wave_sum(sm);
      if (lane == 0) A.l[wave] = A.l[wave] * A.sc[wave] + sm;
    }
    // PV: wave w takes positions w, w+8, ...; lane owns dims [lane*dpl, +dpl)
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      const float scl = h < gs ? A.sc[h] : 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[h][k] *= scl;
    }
    for (int t = wave; t < nb; t += kWaves) {
      const int j = jb + t;
      float vv[4] = {0.f, 0.f, 0.f, 0.f};
      if (j == pos) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (k < dpl) vv[k] = A.v[lane * dpl + k];
      } else {
        const uint16_t* vr = reinterpret_cast<const uint16_t*>(vc) + (size_t)j * hd + lane * dpl;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (k < dpl) vv[k] = bf16_to_f32(vr[k]);
      }
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h < gs) {
          const float pj = A.pr[h][t];
#pragma unroll
          for (int k = 0; k < 4; ++k) o[h][k] = fmaf(pj, vv[k], o[h][k]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (h < gs && k < dpl) A.o[wave][h * hd + lane * dpl + k] = o[h][k];
  __syncthreads();
  // combine waves in a fixed order
  for (int t = threadIdx.x; t < gs * hd; t += kThreads) {
    float acc = 0.f;
    for (int w = 0; w < kWaves; ++w) acc += A.o[w][t];
    A.o[0][t] = acc;
  }
  __syncthreads();
  if (ns == 1) {
    const uint32_t tag = make_tag(epoch, 6 * l + 3);
    uint64_t* ob = p.xch + p.x.o + (uint64_t)par * p.x.par_o;
    for (int t = threadIdx.x; t < gs * hd / 2; t += kThreads) {
      const int h = (2 * t) / hd;
      const float inv = 1.0f / A.l[h];
      const uint32_t w = f32_to_bf16(A.o[0][2 * t] * inv) | (f32_to_bf16(A.o[0][2 * t + 1] * inv) << 16);
      publish(ob, p.x.rep_o, p.R, g * gs * hd / 2 + t, w, tag);
    }
  } else {
    const uint32_t tag = make_tag(epoch, 6 * l + 3);
    uint64_t* pb = p.xch + p.x.part + (uint64_t)par * p.x.par_part;
    for (int t = threadIdx.x; t < gs * (hd + 2); t += kThreads) {
      const int h = t / (hd + 2), k = t - h * (hd + 2);
      const float v = k == 0 ? A.m[h] : (k == 1 ? A.l[h] : A.o[0][h * hd + k - 2]);
      const uint64_t idx = ((uint64_t)(g * gs + h) * p.ns_max + sidx) * (hd + 2) + k;
      st_word(pb + idx, ((uint64_t)__float_as_uint(v) << 32) | tag);
    }
  }
  return true;
}

// Merge the splits of q head h: M = max m_s, L = sum l_s e^(m_s-M),
// o = sum o_s e^(m_s-M) / L.
__device__ __forceinline__ bool merge_unit(const Params& p, Smem& s, int l, int h, int ns, uint32_t epoch) {
  const int hd = p.hd, par = l & 1;
  const uint32_t tag = make_tag(epoch, 6 * l + 3);
  const uint64_t* pb = p.xch + p.x.part + (uint64_t)par * p.x.par_part + (uint64_t)h * p.ns_max * (hd + 2);
  const bool ok = gather(pb, ns * (hd + 2), tag, s.vin, p);
  if (__syncthreads_or(!ok)) return false;
  float M = -INFINITY;
  for (int k = 0; k < ns; ++k) M = fmaxf(M, __uint_as_float(s.vin[k * (hd + 2)]));
  float L = 0.f;
  for (int k = 0; k < ns; ++k)
    L += __uint_as_float(s.vin[k * (hd + 2) + 1]) * expf(__uint_as_float(s.vin[k * (hd + 2)]) - M);
  const float inv = 1.0f / L;
  const uint32_t tag_o = make_tag(epoch, 6 * l + 4);
  uint64_t* ob = p.xch + p.x.o + (uint64_t)par * p.x.par_o;
  for (int t = threadIdx.x; t < hd / 2; t += kThreads) {
    float a = 0.f, b = 0.f;
    for (int k = 0; k < ns; ++k) {
      const float e = expf(__uint_as_float(s.vin[k * (hd + 2)]) - M);
      a = fmaf(__uint_as_float(s.vin[k * (hd + 2) + 2 + 2 * t]), e, a);
      b = fmaf(__uint_as_float(s.vin[k * (hd + 2) + 3 + 2 * t]), e, b);
    }
    const uint32_t w = f32_to_bf16(a * inv) | (f32_to_bf16(b * inv) << 16);
    publish(ob, p.x.rep_o, p.R, h * hd / 2 + t, w, tag_o);
  }
  return true;
}

// ----------------------------------------------------------------- kernel
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(const Params* __restrict__ pp,
                                                              const int32_t* d_token, int pos, uint32_t epoch,
                                                              int32_t* d_next, float* d_logits) {
  __shared__ Smem s;
  const Params& p = *pp;
  const int G = p.grid, wg = blockIdx.x;
  XrayClock xc;
  const int token = __hip_atomic_load(const_cast<int32_t*>(d_token), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (token < 0 || token >= p.V) {
    if (wg == 0 && threadIdx.x == 0) {
      raise_error(p, ERR_TOKEN);
      *d_next = -1;
    }
    return;
  }
  if (wg == 0 && threadIdx.x == 0) *d_next = -1;  // overwritten on success
  const int H = p.H, hd = p.hd;
  const int nqkv = (p.nq + 2 * p.nkv) * hd;
  int oa, ob;
  split_range(H, G, wg, oa, ob);
  const int nown = ob - oa;
  const int rep = wg % p.R;

  // ---- embedding: this workgroup's residual rows
  XR_BEGIN(xc);
  {
    const uint32_t tag = make_tag(epoch, 1);
    uint64_t* xd = p.xch + p.x.x_d + 1 * p.x.par_x;  // parity of layer -1
    for (int i = threadIdx.x; i < nown; i += kThreads) {
      const uint64_t e = (uint64_t)token * H + oa + i;
      float v;
      if (p.embed.fmt == FMT_BF16) v = bf16_to_f32(reinterpret_cast<const uint16_t*>(p.w + p.embed.codes)[e]);
      else v = e4m3_to_f32(p.w[p.embed.codes + e]) *
               reinterpret_cast<const float*>(p.w + p.embed.scales)[token];
      s.x_own[i] = v;
      publish(xd, p.x.rep_x, p.R, oa + i, __float_as_uint(v), tag);
    }
  }
  XR_END(xc, p, 1);

  int ns, span;
  att_split(p, pos + 1, ns, span);

  for (int l = 0; l < p.L; ++l) {
    const uint64_t loff = (uint64_t)l * p.layer_stride;
    const int par = l & 1;
    const Layer& L0 = p.layer0;
    // ---- QKV
    {
      XR_BEGIN(xc);
      const Mat m = at_layer(L0.qkv, loff);
      int ra, rb;
      split_range(nqkv, G, wg, ra, rb);
      const uint64_t* src = p.xch + p.x.x_d + (uint64_t)((l + 1) & 1) * p.x.par_x + (uint64_t)rep * p.x.rep_x;
      if (!gemv_phase(p, s, m, ra, rb - ra, src, H, make_tag(epoch, 6 * l + 1), L0.in_norm + loff, xc)) return;
      const uint32_t tag = make_tag(epoch, 6 * l + 2);
      uint64_t* dst = p.xch + p.x.qkv + (uint64_t)par * p.x.par_qkv;
      for (int t = threadIdx.x; t < rb - ra; t += kThreads)
        publish(dst, p.x.rep_qkv, p.R, ra + t, __float_as_uint(s.u.g.y[t]), tag);
      XR_END(xc, p, 6 * l + 2);
    }
    // ---- attention
    {
      XR_BEGIN(xc);
      for (int u = wg; u < p.nkv * ns; u += G) {
        XR_ACTIVE(xc);
        if (!attention_unit(p, s, l, u / ns, u % ns, ns, span, pos, epoch)) return;
        __syncthreads();
      }
      XR_END(xc, p, 6 * l + 3);
    }
    // ---- merge of position splits
    {
      XR_BEGIN(xc);
      if (ns > 1) {
        for (int h = wg; h < p.nq; h += G) {
          XR_ACTIVE(xc);
          if (!merge_unit(p, s, l, h, ns, epoch)) return;
          __syncthreads();
        }
      }
      XR_END(xc, p, 6 * l + 4);
    }
    // ---- O-projection + residual
    {
      XR_BEGIN(xc);
      const Mat m = at_layer(L0.o, loff);
      const uint64_t* src = p.xch + p.x.o + (uint64_t)par * p.x.par_o + (uint64_t)rep * p.x.rep_o;
      const uint32_t tag_in = make_tag(epoch, ns > 1 ? 6 * l + 4 : 6 * l + 3);
      if (!gemv_phase(p, s, m, oa, nown, src, p.nq * hd / 2, tag_in, 0, xc)) return;
      const uint32_t tag = make_tag(epoch, 6 * l + 5);
      uint64_t* dst = p.xch + p.x.x_o + (uint64_t)par * p.x.par_x;
      for (int t = threadIdx.x; t < nown; t += kThreads) {
        s.x_own[t] += s.u.g.y[t];
        publish(dst, p.x.rep_x, p.R, oa + t, __float_as_uint(s.x_own[t]), tag);
      }
      XR_END(xc, p, 6 * l + 5);
    }
    // ---- gate/up + SwiGLU
    {
      XR_BEGIN(xc);
      const Mat m = at_layer(L0.gu, loff);
      int pa, pb;
      split_range(p.I / 2, G, wg, pa, pb);
      const uint64_t* src = p.xch + p.x.x_o + (uint64_t)par * p.x.par_x + (uint64_t)rep * p.x.rep_x;
      if (!gemv_phase(p, s, m, 4 * pa, 4 * (pb - pa), src, H, make_tag(epoch, 6 * l + 5), L0.post_norm + loff, xc))
        return;
      const uint32_t tag = make_tag(epoch, 6 * l + 6);
      uint64_t* dst = p.xch + p.x.h + (uint64_t)par * p.x.par_h;
      for (int t = threadIdx.x; t < pb - pa; t += kThreads) {
        const float* y = s.u.g.y + 4 * t;
        const float h0 = (y[0] / (1.0f + expf(-y[0]))) * y[1];
        const float h1 = (y[2] / (1.0f + expf(-y[2]))) * y[3];
        publish(dst, p.x.rep_h, p.R, pa + t, f32_to_bf16(h0) | (f32_to_bf16(h1) << 16), tag);
      }
      XR_END(xc, p, 6 * l + 6);
    }
    // ---- down + residual
    {
      XR_BEGIN(xc);
      const Mat m = at_layer(L0.down, loff);
      const uint64_t* src = p.xch + p.x.h + (uint64_t)par * p.x.par_h + (uint64_t)rep * p.x.rep_h;
      if (!gemv_phase(p, s, m, oa, nown, src, p.I / 2, make_tag(epoch, 6 * l + 6), 0, xc)) return;
      const uint32_t tag = make_tag(epoch, 6 * l + 7);
      uint64_t* dst = p.xch + p.x.x_d + (uint64_t)par * p.x.par_x;
      for (int t = threadIdx.x; t < nown; t += kThreads) {
        s.x_own[t] += s.u.g.y[t];
        publish(dst, p.x.rep_x, p.R, oa + t, __float_as_uint(s.x_own[t]), tag);
      }
      XR_END(xc, p, 6 * l + 7);
    }
  }

  // ---- final RMSNorm + tied LM head + this workgroup's argmax
  const int ph_head = 6 * p.L + 2;
  {
    XR_BEGIN(xc);
    int va, vb;
    split_range(p.V, G, wg, va, vb);
    const uint64_t* src = p.xch + p.x.x_d + (uint64_t)((p.L - 1) & 1) * p.x.par_x + (uint64_t)rep * p.x.rep_x;
    if (!gemv_phase(p, s, p.embed, va, vb - va, src, H, make_tag(epoch, 6 * p.L + 1), p.final_norm, xc)) return;
    float best = -INFINITY;
    int bidx = 0x7FFFFFFF;
    for (int t = threadIdx.x; t < vb - va; t += kThreads) {
      const float v = s.u.g.y[t];
      if (d_logits) d_logits[va + t] = v;
      if (v > best) {  // rows ascend within a thread, so the first maximum is kept
        best = v;
        bidx = va + t;
      }
    }
    // workgroup argmax: largest value, then smallest index
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o);
      const int oi = __shfl_xor(bidx, o);
      if (ov > best || (ov == best && oi < bidx)) {
        best = ov;
        bidx = oi;
      }
    }
    if ((threadIdx.x & 63) == 0) {
      s.red[threadIdx.x >> 6] = best;
      s.redi[threadIdx.x >> 6] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < kWaves; ++w)
        if (s.red[w] > best || (s.red[w] == best && s.redi[w] < bidx)) {
          best = s.red[w];
          bidx = s.redi[w];
        }
      const uint32_t tag = make_tag(epoch, ph_head);
      uint64_t* a = p.xch + p.x.arg + 2ull * wg;
      st_word(a, ((uint64_t)__float_as_uint(best) << 32) | tag);
      st_word(a + 1, ((uint64_t)(uint32_t)bidx << 32) | tag);
    }
    XR_END(xc, p, ph_head);
  }
  // ---- workgroup 0 reduces the per-workgroup winners
  if (wg == 0) {
    XR_BEGIN(xc);
    XR_ACTIVE(xc);
    XR_WAIT_BEGIN(xc);
    const bool ok = gather(p.xch + p.x.arg, 2 * G, make_tag(epoch, ph_head), s.vin, p);
    if (__syncthreads_or(!ok)) return;
    XR_WAIT_END(xc);
    float best = -INFINITY;
    int bidx = 0x7FFFFFFF;
    for (int t = threadIdx.x; t < G; t += kThreads) {
      const float v = __uint_as_float(s.vin[2 * t]);
      const int i = (int)s.vin[2 * t + 1];
      if (v > best || (v == best && i < bidx)) {
        best = v;
        bidx = i;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o);
      const int oi = __shfl_xor(bidx, o);
      if (ov > best || (ov == best && oi < bidx)) {
        best = ov;
        bidx = oi;
      }
    }
    if ((threadIdx.x & 63) == 0) {
      s.red[threadIdx.x >> 6] = best;
      s.redi[threadIdx.x >> 6] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < kWaves; ++w)
        if (s.red[w] > best || (s.red[w] == best && s.redi[w] < bidx)) {
          best = s.red[w];
          bidx = s.redi[w];
        }
      *d_next = bidx;
    }
    XR_END(xc, p, ph_head + 1);
  }
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
  v = wave_max(v);
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

// NVFP4: ts = A/2688 (1 if A = 0); per 16-block bs = e4m3(a_b/fl32(6 ts)),
// eff = e4m3(bs) * ts, c = e2m1(w/eff) (all 0 when eff = 0).  One thread per block.
__global__ void pack_fp4_kernel(const uint16_t* src, int N, int K, uint8_t* codes, uint8_t* bscales, float* tscale,
                                int ts_index, const uint32_t* amax, int row_off, int row_step) {
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
    const uint32_t bs = f32_to_e4m3(ab / six_ts);
    const float eff = e4m3_to_f32(bs) * ts;
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
  if (codec == 0) {
    out[i] = e4m3_to_f32(in[i]);
  } else {
    float f[8];
    e2m1x8_to_f32((uint32_t)(in[i] & 0xF), f);
    out[i] = f[0];
  }
}

// ------------------------------------------------------- launch wrappers
hipError_t launch_decode(const Params* d_params, int grid, const int32_t* d_token, int pos, uint32_t epoch,
                         int32_t* d_next, float* d_logits, hipStream_t s) {
  void* args[] = {&d_params, &d_token, &pos, &epoch, &d_next, &d_logits};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(decode_kernel), dim3(grid), dim3(kThreads),
                                    args, 0, s);
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
                           int ts_index, uint32_t* amax, int row_off, int row_step, hipStream_t s) {
  hipError_t e = hipMemsetAsync(amax, 0, 4, s);
  if (e != hipSuccess) return e;
  const size_t n = (size_t)N * K;
  hipLaunchKernelGGL(amax_kernel, dim3(1024), dim3(256), 0, s, src, n, amax);
  hipLaunchKernelGGL(pack_fp4_kernel, dim3(N), dim3(64), 0, s, src, N, K, codes, bscales, tscale, ts_index, amax,
                     row_off, row_step);
  return hipGetLastError();
}

hipError_t launch_rope(float* out, int max_ctx, int hd, double theta, hipStream_t s) {
  hipLaunchKernelGGL(rope_kernel, dim3(1024), dim3(256), 0, s, out, max_ctx, hd, theta);
  return hipGetLastError();
}

hipError_t launch_decode_codes(int codec, const uint8_t* in, int n, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_codes_kernel, dim3((n + 255) / 256), dim3(256), 0, s, codec, in, n, out);
  return hipGetLastError();
}

}  // namespace mk
