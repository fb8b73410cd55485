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

constexpr int kMaxGroupDim = 256;    // (q heads per KV head) * head_dim
constexpr int kMaxGroup = 4;         // q heads per KV head

struct AttSmem {
  float raw[kMaxGroupDim + 256];         // gathered q heads (gs*hd), then k (hd), then v (hd)
  float qw[kWaves][kMaxGroupDim];        // per wave: normed + roped q (wave-private)
  uint32_t kvw[kWaves][128];             // per wave: this position's k (roped) and v as bf16 pairs
  float prow[kWaves][4][kMaxGroupDim];   // per wave: 16-lane-row partial outputs (wave-private)
  float wo[kWaves][kMaxGroupDim];        // per wave: output over its positions
  float wm[kWaves][kMaxGroup], wl[kWaves][kMaxGroup];
};
struct Smem {
  uint32_t vin[kMaxVecWords];            // gathered payloads
  AttSmem att;
  float red[kWaves * 2];
  int32_t redi[kWaves];
  float x_own[kMaxOwn];                  // residual rows this workgroup owns
};

__device__ __forceinline__ void split_range(int n, int parts, int i, int& a, int& b) {
  a = (int)((int64_t)n * i / parts);
  b = (int)((int64_t)n * (i + 1) / parts);
}

// This wave's index, as a value the compiler knows is uniform across the wave.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Cross-lane reductions with DPP (row operations on the VALU) and
// v_readlane, instead of ds_bpermute round trips through the LDS crossbar.
// DPP controls (gfx9): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_ror:4 = 0x124, row_ror:8 = 0x128, row_half_mirror = 0x141.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over the 8-lane group (lanes 8k..8k+7), result in every lane of it.
__device__ __forceinline__ float sum8(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  return v + dpp<0x141>(v);
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x124>(v);
  return v + dpp<0x128>(v);
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  return fmaxf(v, dpp<0x128>(v));
}
__device__ __forceinline__ float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// Sum / max over the wave, the same value in every lane (fixed order).
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = max16(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// ------------------------------------------------------------------ GEMV
// A GEMV phase is wave-autonomous: after the workgroup has gathered the input
// vector, each wave computes the RMSNorm factor itself (the page's
// every-block-recomputes-the-norm trick, taken down to the wave), keeps its
// slice of the activations in registers, and owns whole output units (one
// row, or for gate/up the four rows behind one output word), so each unit is
// finished with one DPP reduction and published by the wave that computed
// it: no barrier after the wait.
//
// Lane l covers elements [c*1024 + 16 l, +16) of every row for chunk c, so a
// wave streams each row as contiguous 1 KB (fp8) / 2 KB (bf16) / 512 B (fp4)
// runs with 16-byte (fp4: 8-byte) loads.  Units u = wave + 8 j; a wave keeps
// UB units' weights in registers, double-buffered.

// One matrix of one phase, with its pointers resolved once.
struct GMat {
  MK_GLOBAL const uint8_t* codes;
  MK_GLOBAL const uint8_t* scales;  // fp8: fp32 per row; fp4: e4m3 per 16-block
  MK_GLOBAL const float* ts;        // fp4: tensor scales
  uint32_t K, ts_mode, ts_b0, ts_b1;
};

__device__ __forceinline__ GMat gmat(MK_GLOBAL const uint8_t* W, const Mat& m, uint64_t off) {
  GMat g;
  g.codes = W + m.codes + off;
  g.scales = W + m.scales + off;
  g.ts = GCAST(const float, W + m.tscale + off);
  g.K = m.K;
  g.ts_mode = m.ts_mode;
  g.ts_b0 = m.ts_b0;
  g.ts_b1 = m.ts_b1;
  return g;
}

__device__ __forceinline__ float fp4_tensor_scale(const GMat& g, uint32_t row) {
  uint32_t idx = 0;
  if (g.ts_mode == 1) idx = row < g.ts_b0 ? 0u : (row < g.ts_b1 ? 1u : 2u);
  else if (g.ts_mode == 2) idx = row & 1u;
  return g.ts[idx];
}

template <uint32_t FMT, int NCH, int UR, int UB>
struct WBatch {
  v4u a[UB][UR][NCH];   // bf16: first 16 B; fp8: 16 B; fp4: 8 B codes in .xy
  v4u b[UB][UR][NCH];   // bf16: second 16 B; fp4: block-scale byte in .x
  float rs[UB][UR];     // fp8 row scale / fp4 tensor scale
};

// Load units j0 .. j0+UB-1 of this wave.  Indices are clamped instead of
// guarded, so no load sits behind a branch (a guarded load ends in a wait
// that would drain every load in flight); clamped lanes and units are
// discarded later.
template <uint32_t FMT, int NCH, int UR, int UB>
__device__ __forceinline__ void wload(const GMat& g, int r0, int nunits, int wave, int j0,
                                      WBatch<FMT, NCH, UR, UB>& B) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int ub = 0; ub < UB; ++ub) {
    const int u = min(wave + kWaves * (j0 + ub), nunits - 1);
#pragma unroll
    for (int r = 0; r < UR; ++r) {
      const uint32_t row = (uint32_t)(r0 + u * UR + r);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t e0 = (uint32_t)min(c * 1024 + 16 * lane, (int)g.K - 16);
        const uint32_t el = row * g.K + e0;
        if (FMT == FMT_BF16) {
          MK_GLOBAL const v4u* q = GCAST(const v4u, g.codes + 2ull * el);
          B.a[ub][r][c] = q[0];
          B.b[ub][r][c] = q[1];
        } else if (FMT == FMT_FP8) {
          B.a[ub][r][c] = *GCAST(const v4u, g.codes + el);
        } else {
          const v2u c2 = *GCAST(const v2u, g.codes + el / 2);
          B.a[ub][r][c].x = c2.x;
          B.a[ub][r][c].y = c2.y;
          B.b[ub][r][c].x = g.scales[el / 16];
        }
      }
      if (FMT == FMT_FP8) B.rs[ub][r] = GCAST(const float, g.scales)[row];
      if (FMT == FMT_FP4) B.rs[ub][r] = fp4_tensor_scale(g, row);
    }
  }
}

// Dot products of units j0.. with the activations xa; epi(u, vals) per unit.
template <uint32_t FMT, int NCH, int UR, int UB, class Epi>
__device__ __forceinline__ void wcompute(const WBatch<FMT, NCH, UR, UB>& B, const uint32_t (&xa)[NCH][8],
                                         int nunits, int wave, int j0, Epi& epi) {
#pragma unroll
  for (int ub = 0; ub < UB; ++ub) {
    const int u = wave + kWaves * (j0 + ub);
    if (u >= nunits) break;  // uniform
    float vals[UR];
#pragma unroll
    for (int r = 0; r < UR; ++r) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t* xs = xa[c];
        float ac = 0.f;
        if (FMT == FMT_BF16) {
          const uint32_t ws[8] = {B.a[ub][r][c].x, B.a[ub][r][c].y, B.a[ub][r][c].z, B.a[ub][r][c].w,
                                  B.b[ub][r][c].x, B.b[ub][r][c].y, B.b[ub][r][c].z, B.b[ub][r][c].w};
#pragma unroll
          for (int j = 0; j < 8; ++j) ac = dot2(ws[j], xs[j], ac);
        } else if (FMT == FMT_FP8) {
          const uint32_t ws[4] = {B.a[ub][r][c].x, B.a[ub][r][c].y, B.a[ub][r][c].z, B.a[ub][r][c].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ac = dot2(e4m3x2_to_bf16x2<false>(ws[j]), xs[2 * j], ac);
            ac = dot2(e4m3x2_to_bf16x2<true>(ws[j]), xs[2 * j + 1], ac);
          }
        } else {
          const uint32_t ws[2] = {B.a[ub][r][c].x, B.a[ub][r][c].y};
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            ac = dot2(e2m1x2_to_bf16x2<0>(ws[j]), xs[4 * j + 0], ac);
            ac = dot2(e2m1x2_to_bf16x2<1>(ws[j]), xs[4 * j + 1], ac);
            ac = dot2(e2m1x2_to_bf16x2<2>(ws[j]), xs[4 * j + 2], ac);
            ac = dot2(e2m1x2_to_bf16x2<3>(ws[j]), xs[4 * j + 3], ac);
          }
          ac *= e4m3_to_f32(B.b[ub][r][c].x);   // the lane's chunk is one 16-block
        }
        a += ac;
      }
      a = wave_sum(a);
      if (FMT != FMT_BF16) a *= B.rs[ub][r];
      vals[r] = a;
    }
    epi(u, vals);
  }
}

// A GEMV phase: gains and the first weight batch are loaded before the wait
// for the input vector; then the wave's units are computed in double-buffered
// batches.  NORM: the input is the fp32 residual and is RMSNormed (gains
// `gain`) and rounded to bf16; otherwise it is already bf16 pairs.
template <uint32_t FMT, int NCH, int UR, int UB, bool NORM, class Epi>
__device__ __forceinline__ bool gemv_phase(const Params& p, Smem& s, const GMat& g, int r0, int nunits,
                                           MK_GLOBAL const uint64_t* src, int nwords, uint32_t tag,
                                           MK_GLOBAL const uint32_t* gain, XrayClock& xc, Epi epi) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int nj = nunits > wave ? (nunits - wave + kWaves - 1) / kWaves : 0;  // units of this wave
  uint32_t gn[NCH][8];
  if (NORM) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = min(c * 1024 + 16 * lane, (int)g.K - 16);
      MK_GLOBAL const v4u* gp = GCAST(const v4u, gain + e0 / 2);
      const v4u g0 = gp[0], g1 = gp[1];
      gn[c][0] = g0.x; gn[c][1] = g0.y; gn[c][2] = g0.z; gn[c][3] = g0.w;
      gn[c][4] = g1.x; gn[c][5] = g1.y; gn[c][6] = g1.z; gn[c][7] = g1.w;
    }
  }
  WBatch<FMT, NCH, UR, UB> B0, B1;
  if (nj > 0) wload(g, r0, nunits, wave, 0, B0);
  // Compiler memory barrier: keeps the loads above issued before the wait.
  // Without it they may legally sink to their first use after the wait (the
  // wait touches only LDS and atomics the weights cannot alias), and every
  // phase would pay the weight latency after its input arrives.  It reads no
  // register, so it adds no wait of its own.
  asm volatile("" ::: "memory");
  XR_WAIT_BEGIN(xc);
  const bool ok = gather(src, nwords, tag, s.vin, p);
  if (__syncthreads_or(!ok)) return false;
  XR_WAIT_END(xc);
  if (nj <= 0) return true;
  XR_ACTIVE(xc);
  uint32_t xa[NCH][8];
  if (NORM) {
    float x[NCH][16];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = c * 1024 + 16 * lane;
      const bool in = e0 < (int)g.K;
      const v4u* xp = reinterpret_cast<const v4u*>(s.vin + min(e0, (int)g.K - 16));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4u w = xp[q];
        x[c][4 * q + 0] = in ? __uint_as_float(w.x) : 0.f;
        x[c][4 * q + 1] = in ? __uint_as_float(w.y) : 0.f;
        x[c][4 * q + 2] = in ? __uint_as_float(w.z) : 0.f;
        x[c][4 * q + 3] = in ? __uint_as_float(w.w) : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(x[c][i], x[c][i], ss);
    }
    const float r = 1.0f / sqrtf(wave_sum(ss) / (float)g.K + p.eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float lo = bf16_lo(gn[c][j]) * (x[c][2 * j] * r);
        const float hi = bf16_hi(gn[c][j]) * (x[c][2 * j + 1] * r);
        xa[c][j] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
      }
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = c * 1024 + 16 * lane;
      const bool in = e0 < (int)g.K;
      const v4u* xp = reinterpret_cast<const v4u*>(s.vin + min(e0, (int)g.K - 16) / 2);
      const v4u w0 = xp[0], w1 = xp[1];
      xa[c][0] = in ? w0.x : 0u; xa[c][1] = in ? w0.y : 0u; xa[c][2] = in ? w0.z : 0u; xa[c][3] = in ? w0.w : 0u;
      xa[c][4] = in ? w1.x : 0u; xa[c][5] = in ? w1.y : 0u; xa[c][6] = in ? w1.z : 0u; xa[c][7] = in ? w1.w : 0u;
    }
  }
  XR_MARK(xc, 0);
  // the scheduling barriers keep each next batch's loads ahead of the current
  // batch's arithmetic (under register pressure the scheduler would otherwise
  // sink them and serialize the stream)
  for (int jb = 0; jb < nj; jb += 2 * UB) {
    if (jb + UB < nj) wload(g, r0, nunits, wave, jb + UB, B1);
    __builtin_amdgcn_sched_barrier(0);
    wcompute(B0, xa, nunits, wave, jb, epi);
    if (jb + UB >= nj) break;
    if (jb + 2 * UB < nj) wload(g, r0, nunits, wave, jb + 2 * UB, B0);
    __builtin_amdgcn_sched_barrier(0);
    wcompute(B1, xa, nunits, wave, jb + UB, epi);
  }
  XR_MARK(xc, 1);
  return true;
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

// One unit = (KV head g, position split [j0, j1)) on one workgroup.  Eight
// threads share a position (HD/8 dims each); wave w takes positions
// jb + 8w .. jb + 8w + 7 of every 64-position pass, so a wave reads eight
// consecutive cache rows as one coalesced run.  The rows of positions before
// `pos` are already in the cache, so the first pass is loaded before waiting
// for this step's q/k/v and each later pass while the previous one is used.
// Each wave norms and ropes q and k itself (in wave-private LDS) and keeps its
// own online softmax over its positions; one barrier at the end merges the
// eight waves.  The result is the final output (one split) or (max, sum,
// unnormalized output) for the merge phase.
template <int HD, int GS>
__device__ __forceinline__ bool attention_unit_t(const Params& p, Smem& s, int l, int g, int sidx, int ns,
                                                 int span, int pos, uint32_t epoch, XrayClock& xc) {
  constexpr int TPP = 8;              // threads per position
  constexpr int DPT = HD / TPP;       // dims per thread
  constexpr int WPT = DPT / 2;        // bf16 pairs per thread
  constexpr int PPP = kThreads / TPP; // positions per pass
  constexpr int NOUT = GS * HD;       // outputs of the unit
  static_assert(NOUT <= kMaxGroupDim && HD <= 128, "attention shape");
  AttSmem& A = s.att;
  const int nq = p.nq, nkv = p.nkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int pl = lane >> 3, c = lane & 7;
  const int j0 = sidx * span, j1 = min(j0 + span, pos + 1);
  const int par = l & 1;
  const size_t plane = (size_t)p.max_ctx * HD;
  MK_GLOBAL uint32_t* kc = GCAST(uint32_t, p.kv + ((size_t)(l * 2 + 0) * nkv + g) * plane);
  MK_GLOBAL uint32_t* vc = GCAST(uint32_t, p.kv + ((size_t)(l * 2 + 1) * nkv + g) * plane);

  uint32_t kr[WPT], vr[WPT], kn[WPT], vn[WPT];
  // Clamped loads (no guarded loads); positions past the split, and `pos`
  // itself (not yet in the cache: substituted later), become exact zeros so
  // they add nothing, whatever the cache memory held.
  auto load_kv = [&](int jb, uint32_t* kk, uint32_t* vv) {
    const int jr = jb + wave * 8 + pl;
    const int j = min(jr, j1 - 1);
    const bool use = jr < j1 && jr != pos;
    MK_GLOBAL const v4u* kp = GCAST(const v4u, kc + (size_t)j * (HD / 2) + c * WPT);
    MK_GLOBAL const v4u* vp = GCAST(const v4u, vc + (size_t)j * (HD / 2) + c * WPT);
#pragma unroll
    for (int w = 0; w < WPT / 4; ++w) {
      const v4u a = kp[w], b = vp[w];
      kk[4 * w] = use ? a.x : 0u; kk[4 * w + 1] = use ? a.y : 0u;
      kk[4 * w + 2] = use ? a.z : 0u; kk[4 * w + 3] = use ? a.w : 0u;
      vv[4 * w] = use ? b.x : 0u; vv[4 * w + 1] = use ? b.y : 0u;
      vv[4 * w + 2] = use ? b.z : 0u; vv[4 * w + 3] = use ? b.w : 0u;
    }
  };
  load_kv(j0, kr, vr);
  // q/k-norm gains and this position's RoPE pair (lane i < HD/2 owns pair i)
  const Layer& L0 = p.layer0;
  const uint64_t loff = (uint64_t)l * p.layer_stride;
  const int li = min(lane, HD / 2 - 1);
  MK_GLOBAL const uint16_t* gq = GCAST(const uint16_t, p.w + L0.q_norm + loff);
  MK_GLOBAL const uint16_t* gk = GCAST(const uint16_t, p.w + L0.k_norm + loff);
  const float gq_lo = bf16_to_f32(gq[li]), gq_hi = bf16_to_f32(gq[li + HD / 2]);
  const float gk_lo = bf16_to_f32(gk[li]), gk_hi = bf16_to_f32(gk[li + HD / 2]);
  MK_GLOBAL const float* cs = p.rope + ((size_t)pos * (HD / 2) + li) * 2;
  const float rc = cs[0], rsn = cs[1];
  asm volatile("" ::: "memory");  // keep the K/V, gain and RoPE loads ahead of the wait

  // this step's q, k, v of the group, in one gather
  const uint32_t tag_qkv = make_tag(epoch, 6 * l + 2);
  MK_GLOBAL const uint64_t* qkv = p.xch + p.x.qkv + (uint64_t)par * p.x.par_qkv + (uint64_t)(blockIdx.x % p.R) * p.x.rep_qkv;
  const int qo = g * NOUT, ko = (nq + g) * HD, vo = (nq + nkv + g) * HD;
  XR_WAIT_BEGIN(xc);
  const bool ok = gather_map(qkv, NOUT + 2 * HD, tag_qkv, reinterpret_cast<uint32_t*>(A.raw), p,
                             [=](int i) { return i < NOUT ? qo + i : (i < NOUT + HD ? ko + i - NOUT : vo + i - NOUT - HD); });
  if (__syncthreads_or(!ok)) return false;
  XR_WAIT_END(xc);

  // every wave: RMSNorm + RoPE of the q heads and k (lane i < HD/2: pair i)
  const bool pair_lane = lane < HD / 2;
  float* qw = A.qw[wave];
  uint32_t* kvw = A.kvw[wave];
#pragma unroll
  for (int h = 0; h <= GS; ++h) {
    const float* src = A.raw + h * HD;
    const float xa = pair_lane ? src[li] : 0.f, xb = pair_lane ? src[li + HD / 2] : 0.f;
    const float r = 1.0f / sqrtf(wave_sum(xa * xa + xb * xb) / (float)HD + p.eps);
    const float glo = h < GS ? gq_lo : gk_lo, ghi = h < GS ? gq_hi : gk_hi;
    const float a = glo * (xa * r), b = ghi * (xb * r);
    const float ra = a * rc - b * rsn, rb = b * rc + a * rsn;
    if (h < GS) {
      if (pair_lane) {
        qw[h * HD + li] = ra;
        qw[h * HD + li + HD / 2] = rb;
      }
    } else if (pair_lane) {
      // bf16 k as the cache holds it: pairs (2t, 2t+1) are packed below
      A.prow[wave][0][li] = ra;
      A.prow[wave][0][li + HD / 2] = rb;
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < HD / 2) {
    const float* kf = A.prow[wave][0];
    kvw[lane] = f32_to_bf16(kf[2 * lane]) | (f32_to_bf16(kf[2 * lane + 1]) << 16);
    const float* vf = A.raw + (GS + 1) * HD;
    kvw[HD / 2 + lane] = f32_to_bf16(vf[2 * lane]) | (f32_to_bf16(vf[2 * lane + 1]) << 16);
  }
  __builtin_amdgcn_wave_barrier();
  if (wave == 0 && j0 <= pos && pos < j1 && lane < HD / 2) {
    kc[(size_t)pos * (HD / 2) + lane] = kvw[lane];
    vc[(size_t)pos * (HD / 2) + lane] = kvw[HD / 2 + lane];
  }
  // q pre-scaled by log2(e)/sqrt(HD): scores come out in log2 units, so every
  // exponential below is one v_exp_f32 (exp2); the unit's max is kept in the
  // same units for the merge
  const float kq = 1.4426950408889634f / sqrtf((float)HD);
  float qr[GS][DPT];
#pragma unroll
  for (int h = 0; h < GS; ++h)
#pragma unroll
    for (int e = 0; e < DPT; ++e) qr[h][e] = qw[h * HD + c * DPT + e] * kq;
  XR_MARK(xc, 0);

  float acc[GS][DPT];
  float mrun[GS], lrun[GS];
#pragma unroll
  for (int h = 0; h < GS; ++h) {
    mrun[h] = -INFINITY;
    lrun[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[h][e] = 0.f;
  }
  for (int jb = j0; jb < j1; jb += PPP) {
    const bool more = jb + PPP < j1;
    if (more) load_kv(jb + PPP, kn, vn);
    const int j = jb + wave * 8 + pl;
    const bool act = j < j1;
    if (act && j == pos) {
#pragma unroll
      for (int w = 0; w < WPT; ++w) {
        kr[w] = kvw[c * WPT + w];
        vr[w] = kvw[HD / 2 + c * WPT + w];
      }
    }
#pragma unroll
    for (int h = 0; h < GS; ++h) {
      float d = 0.f;
#pragma unroll
      for (int w = 0; w < WPT; ++w) {
        d = fmaf(qr[h][2 * w], bf16_lo(kr[w]), d);
        d = fmaf(qr[h][2 * w + 1], bf16_hi(kr[w]), d);
      }
      const float sc = act ? sum8(d) : -INFINITY;
      const float mn = fmaxf(mrun[h], wave_max(sc));
      if (mn == -INFINITY) continue;   // no position of this wave yet (uniform)
      const float scale = __builtin_amdgcn_exp2f(mrun[h] - mn);
      const float pr = act ? __builtin_amdgcn_exp2f(sc - mn) : 0.f;
      mrun[h] = mn;
      lrun[h] = lrun[h] * scale + wave_sum(c == 0 ? pr : 0.f);
#pragma unroll
      for (int w = 0; w < WPT; ++w) {
        acc[h][2 * w] = fmaf(pr, bf16_lo(vr[w]), acc[h][2 * w] * scale);
        acc[h][2 * w + 1] = fmaf(pr, bf16_hi(vr[w]), acc[h][2 * w + 1] * scale);
      }
    }
    if (more) {
#pragma unroll
      for (int w = 0; w < WPT; ++w) {
        kr[w] = kn[w];
        vr[w] = vn[w];
      }
    }
  }
  // this wave's output: sum over its 8 positions (lanes with the same c):
  // the two 8-lane halves of each 16-lane row with one DPP step, then the
  // four rows through wave-private LDS
#pragma unroll
  for (int h = 0; h < GS; ++h)
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[h][e] += dpp<0x128>(acc[h][e]);
  if ((lane & 8) == 0) {
#pragma unroll
    for (int h = 0; h < GS; ++h)
#pragma unroll
      for (int e = 0; e < DPT; ++e) A.prow[wave][lane >> 4][h * HD + c * DPT + e] = acc[h][e];
  }
  __builtin_amdgcn_wave_barrier();
  for (int t = lane; t < NOUT; t += 64)
    A.wo[wave][t] = (A.prow[wave][0][t] + A.prow[wave][1][t]) + (A.prow[wave][2][t] + A.prow[wave][3][t]);
  if (lane < GS) {
    float mh = mrun[0], lh = lrun[0];
#pragma unroll
    for (int h = 1; h < GS; ++h)
      if (lane == h) {
        mh = mrun[h];
        lh = lrun[h];
      }
    A.wm[wave][lane] = mh;
    A.wl[wave][lane] = lh;
  }
  XR_MARK(xc, 1);
  __syncthreads();
  // merge the eight waves (fixed order)
  const uint32_t tag = make_tag(epoch, 6 * l + 3);
  for (int t = tid; t < NOUT; t += kThreads) {
    const int h = t / HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, A.wm[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = A.wm[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(A.wm[w][h] - M);
      L = fmaf(A.wl[w][h], e, L);
      O = fmaf(A.wo[w][t], e, O);
    }
    if (ns == 1) {
      // final output: pairs of consecutive dims form one bf16-pair word
      const float o = O / L;
      const float o1 = __shfl_xor(o, 1);
      if ((t & 1) == 0) {
        MK_GLOBAL uint64_t* ob = p.xch + p.x.o + (uint64_t)par * p.x.par_o;
        publish(ob, p.x.rep_o, p.R, (g * NOUT + t) / 2, f32_to_bf16(o) | (f32_to_bf16(o1) << 16), tag);
      }
    } else {
      MK_GLOBAL uint64_t* pb = p.xch + p.x.part + (uint64_t)par * p.x.par_part;
      const uint64_t base = ((uint64_t)(g * GS + h) * p.ns_max + sidx) * (HD + 2);
      st_word(pb + base + 2 + (t - h * HD), ((uint64_t)__float_as_uint(O) << 32) | tag);
      if (t - h * HD == 0) {
        st_word(pb + base, ((uint64_t)__float_as_uint(M) << 32) | tag);
        st_word(pb + base + 1, ((uint64_t)__float_as_uint(L) << 32) | tag);
      }
    }
  }
  XR_MARK(xc, 2);
  return true;
}

// Merge the splits of q head h (maxima in log2 units): M = max m_s,
// L = sum l_s 2^(m_s-M), o = sum o_s 2^(m_s-M) / L.
__device__ __forceinline__ bool merge_unit(const Params& p, Smem& s, int l, int h, int ns, uint32_t epoch) {
  const int hd = p.hd, par = l & 1;
  const uint32_t tag = make_tag(epoch, 6 * l + 3);
  MK_GLOBAL const uint64_t* pb = p.xch + p.x.part + (uint64_t)par * p.x.par_part + (uint64_t)h * p.ns_max * (hd + 2);
  const bool ok = gather(pb, ns * (hd + 2), tag, s.vin, p);
  if (__syncthreads_or(!ok)) return false;
  float M = -INFINITY;
  for (int k = 0; k < ns; ++k) M = fmaxf(M, __uint_as_float(s.vin[k * (hd + 2)]));
  float L = 0.f;
  for (int k = 0; k < ns; ++k)
    L += __uint_as_float(s.vin[k * (hd + 2) + 1]) * __builtin_amdgcn_exp2f(__uint_as_float(s.vin[k * (hd + 2)]) - M);
  const float inv = 1.0f / L;
  const uint32_t tag_o = make_tag(epoch, 6 * l + 4);
  MK_GLOBAL uint64_t* ob = p.xch + p.x.o + (uint64_t)par * p.x.par_o;
  for (int t = threadIdx.x; t < hd / 2; t += kThreads) {
    float a = 0.f, b = 0.f;
    for (int k = 0; k < ns; ++k) {
      const float e = __builtin_amdgcn_exp2f(__uint_as_float(s.vin[k * (hd + 2)]) - M);
      a = fmaf(__uint_as_float(s.vin[k * (hd + 2) + 2 + 2 * t]), e, a);
      b = fmaf(__uint_as_float(s.vin[k * (hd + 2) + 3 + 2 * t]), e, b);
    }
    const uint32_t w = f32_to_bf16(a * inv) | (f32_to_bf16(b * inv) << 16);
    publish(ob, p.x.rep_o, p.R, h * hd / 2 + t, w, tag_o);
  }
  return true;
}

// ----------------------------------------------------------------- kernel
// One instantiation per (weight format, head_dim, q heads per KV head,
// 1024-chunks of hidden, of n_q_heads*head_dim and of intermediate): the
// formats, the attention shape and every per-lane register array size are
// compile-time constants.
template <int WF, int HD, int GS, int NH, int NQ, int NI>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(const Params* __restrict__ pp,
                                                              const int32_t* d_token, int pos, uint32_t epoch,
                                                              int32_t* d_next, float* d_logits) {
  __shared__ Smem s;
  const Params& p = *pp;
  MK_GLOBAL const uint8_t* const W = p.w;  // held in registers for the whole step
  constexpr uint32_t F_LIN = WF == 0 ? FMT_BF16 : (WF == 1 ? FMT_FP8 : FMT_FP4);  // q, k, v, o, gate, up
  constexpr uint32_t F_8 = WF == 0 ? FMT_BF16 : FMT_FP8;                          // down, embed / LM head
  const int G = p.grid, wg = blockIdx.x;
  const int lane = threadIdx.x & 63;
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
  const int H = p.H, hd = p.hd, R = p.R;
  const int nqkv = (p.nq + 2 * p.nkv) * hd;
  int oa, ob;
  split_range(H, G, wg, oa, ob);
  const int nown = ob - oa;
  const int rep = wg % R;
  // publish by lanes 0..R-1, one replica each
  auto put = [&](MK_GLOBAL uint64_t* base, uint64_t rep_stride, int i, uint32_t payload, uint32_t tag) {
    if (lane < R) st_word(base + (uint64_t)lane * rep_stride + i, ((uint64_t)payload << 32) | tag);
  };

  // ---- embedding: this workgroup's residual rows
  XR_BEGIN(xc);
  {
    const uint32_t tag = make_tag(epoch, 1);
    MK_GLOBAL uint64_t* xd = p.xch + p.x.x_d + 1 * p.x.par_x;  // parity of layer -1
    for (int i = threadIdx.x; i < nown; i += kThreads) {
      const uint64_t e = (uint64_t)token * H + oa + i;
      float v;
      if (F_8 == FMT_BF16) v = bf16_to_f32(GCAST(const uint16_t, W + p.embed.codes)[e]);
      else v = e4m3_to_f32(W[p.embed.codes + e]) * GCAST(const float, W + p.embed.scales)[token];
      s.x_own[i] = v;
      publish(xd, p.x.rep_x, R, oa + i, __float_as_uint(v), tag);
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
      int ra, rb;
      split_range(nqkv, G, wg, ra, rb);
      MK_GLOBAL const uint64_t* src = p.xch + p.x.x_d + (uint64_t)((l + 1) & 1) * p.x.par_x + (uint64_t)rep * p.x.rep_x;
      MK_GLOBAL uint64_t* dst = p.xch + p.x.qkv + (uint64_t)par * p.x.par_qkv;
      const uint32_t tag = make_tag(epoch, 6 * l + 2);
      auto epi = [&](int u, const float* v) { put(dst, p.x.rep_qkv, ra + u, __float_as_uint(v[0]), tag); };
      if (!gemv_phase<F_LIN, NH, 1, 2, true>(p, s, gmat(W, L0.qkv, loff), ra, rb - ra, src, H,
                                            make_tag(epoch, 6 * l + 1), GCAST(const uint32_t, W + L0.in_norm + loff),
                                            xc, epi))
        return;
      XR_MARK(xc, 3);
      XR_END(xc, p, 6 * l + 2);
    }
    // ---- attention
    {
      XR_BEGIN(xc);
      for (int u = wg; u < p.nkv * ns; u += G) {
        XR_ACTIVE(xc);
        if (!attention_unit_t<HD, GS>(p, s, l, u / ns, u % ns, ns, span, pos, epoch, xc)) return;
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
      MK_GLOBAL const uint64_t* src = p.xch + p.x.o + (uint64_t)par * p.x.par_o + (uint64_t)rep * p.x.rep_o;
      MK_GLOBAL uint64_t* dst = p.xch + p.x.x_o + (uint64_t)par * p.x.par_x;
      const uint32_t tag = make_tag(epoch, 6 * l + 5);
      auto epi = [&](int u, const float* v) {
        const float x = s.x_own[u] + v[0];
        s.x_own[u] = x;  // this row belongs to this wave only
        put(dst, p.x.rep_x, oa + u, __float_as_uint(x), tag);
      };
      if (!gemv_phase<F_LIN, NQ, 1, 1, false>(p, s, gmat(W, L0.o, loff), oa, nown, src, p.nq * hd / 2,
                                             make_tag(epoch, ns > 1 ? 6 * l + 4 : 6 * l + 3), nullptr, xc, epi))
        return;
      XR_MARK(xc, 3);
      XR_END(xc, p, 6 * l + 5);
    }
    // ---- gate/up + SwiGLU: a unit is the four rows behind one output word
    {
      XR_BEGIN(xc);
      int pa, pb;
      split_range(p.I / 2, G, wg, pa, pb);
      MK_GLOBAL const uint64_t* src = p.xch + p.x.x_o + (uint64_t)par * p.x.par_x + (uint64_t)rep * p.x.rep_x;
      MK_GLOBAL uint64_t* dst = p.xch + p.x.h + (uint64_t)par * p.x.par_h;
      const uint32_t tag = make_tag(epoch, 6 * l + 6);
      auto epi = [&](int u, const float* y) {
        const float h0 = (y[0] / (1.0f + expf(-y[0]))) * y[1];
        const float h1 = (y[2] / (1.0f + expf(-y[2]))) * y[3];
        put(dst, p.x.rep_h, pa + u, f32_to_bf16(h0) | (f32_to_bf16(h1) << 16), tag);
      };
      if (!gemv_phase<F_LIN, NH, 4, 1, true>(p, s, gmat(W, L0.gu, loff), 4 * pa, pb - pa, src, H,
                                            make_tag(epoch, 6 * l + 5), GCAST(const uint32_t, W + L0.post_norm + loff),
                                            xc, epi))
        return;
      XR_MARK(xc, 3);
      XR_END(xc, p, 6 * l + 6);
    }
    // ---- down + residual
    {
      XR_BEGIN(xc);
      MK_GLOBAL const uint64_t* src = p.xch + p.x.h + (uint64_t)par * p.x.par_h + (uint64_t)rep * p.x.rep_h;
      MK_GLOBAL uint64_t* dst = p.xch + p.x.x_d + (uint64_t)par * p.x.par_x;
      const uint32_t tag = make_tag(epoch, 6 * l + 7);
      auto epi = [&](int u, const float* v) {
        const float x = s.x_own[u] + v[0];
        s.x_own[u] = x;
        put(dst, p.x.rep_x, oa + u, __float_as_uint(x), tag);
      };
      if (!gemv_phase<F_8, NI, 1, 1, false>(p, s, gmat(W, L0.down, loff), oa, nown, src, p.I / 2,
                                           make_tag(epoch, 6 * l + 6), nullptr, xc, epi))
        return;
      XR_MARK(xc, 3);
      XR_END(xc, p, 6 * l + 7);
    }
  }

  // ---- final RMSNorm + tied LM head + this workgroup's argmax
  const int ph_head = 6 * p.L + 2;
  {
    XR_BEGIN(xc);
    int va, vb;
    split_range(p.V, G, wg, va, vb);
    MK_GLOBAL const uint64_t* src = p.xch + p.x.x_d + (uint64_t)((p.L - 1) & 1) * p.x.par_x + (uint64_t)rep * p.x.rep_x;
    float best = -INFINITY;
    int bidx = 0x7FFFFFFF;
    auto epi = [&](int u, const float* v) {
      if (d_logits && lane == 0) d_logits[va + u] = v[0];
      if (v[0] > best) {  // a wave's rows ascend, so the first maximum is kept
        best = v[0];
        bidx = va + u;
      }
    };
    constexpr int UBH = F_8 == FMT_BF16 ? 4 : 8;
    if (!gemv_phase<F_8, NH, 1, UBH, true>(p, s, gmat(W, p.embed, 0), va, vb - va, src, H,
                                          make_tag(epoch, 6 * p.L + 1), GCAST(const uint32_t, W + p.final_norm), xc,
                                          epi))
      return;
    // workgroup argmax: largest value, then smallest index
    if (lane == 0) {
      s.red[wave_id()] = best;
      s.redi[wave_id()] = bidx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      best = s.red[0];
      bidx = s.redi[0];
      for (int w = 1; w < kWaves; ++w)
        if (s.red[w] > best || (s.red[w] == best && s.redi[w] < bidx)) {
          best = s.red[w];
          bidx = s.redi[w];
        }
      const uint32_t tag = make_tag(epoch, ph_head);
      MK_GLOBAL uint64_t* a = p.xch + p.x.arg + 2ull * wg;
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
    if (threadIdx.x < 64) {
      float best = -INFINITY;
      int bidx = 0x7FFFFFFF;
      for (int t = lane; t < G; t += 64) {
        const float v = __uint_as_float(s.vin[2 * t]);
        const int i = (int)s.vin[2 * t + 1];
        if (v > best || (v == best && i < bidx)) {
          best = v;
          bidx = i;
        }
      }
      const float m = wave_max(best);
      const int cand = best == m ? bidx : 0x7FFFFFFF;
      // smallest index among the lanes holding the maximum
      int mi = cand;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mi = min(mi, __shfl_xor(mi, o));
      if (lane == 0) *d_next = mi;
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

// ------------------------------------------------------- launch wrappers
// Compiled shape classes: (head_dim, q heads per KV head, 1024-chunks of
// hidden, of n_q_heads*head_dim, of intermediate); three weight formats each.
// The tiny test decoder and the Qwen3-0.6B shape.
#define MK_SHAPES(X) X(64, 2, 1, 1, 1) X(128, 2, 1, 2, 3)

static int cdiv1024(int n) { return (n + 1023) / 1024; }

bool decode_shape_supported(int hd, int gs, int hidden, int qdim, int inter) {
  const int nh = cdiv1024(hidden), nqd = cdiv1024(qdim), ni = cdiv1024(inter);
#define MK_CASE(H_, G_, A_, B_, C_) if (hd == H_ && gs == G_ && nh == A_ && nqd == B_ && ni == C_) return true;
  MK_SHAPES(MK_CASE)
#undef MK_CASE
  return false;
}

hipError_t launch_decode(const Params* d_params, int wfmt, int hd, int gs, int hidden, int qdim, int inter, int grid,
                         const int32_t* d_token, int pos, uint32_t epoch, int32_t* d_next, float* d_logits,
                         hipStream_t s) {
  const void* fn = nullptr;
  const int nh = cdiv1024(hidden), nqd = cdiv1024(qdim), ni = cdiv1024(inter);
#define MK_CASE(H_, G_, A_, B_, C_)                                                                             \
  if (hd == H_ && gs == G_ && nh == A_ && nqd == B_ && ni == C_) {                                              \
    fn = wfmt == 0 ? reinterpret_cast<const void*>(decode_kernel<0, H_, G_, A_, B_, C_>)                        \
                   : (wfmt == 1 ? reinterpret_cast<const void*>(decode_kernel<1, H_, G_, A_, B_, C_>)           \
                                : reinterpret_cast<const void*>(decode_kernel<2, H_, G_, A_, B_, C_>));         \
  }
  MK_SHAPES(MK_CASE)
#undef MK_CASE
  if (!fn) return hipErrorInvalidValue;
  void* args[] = {&d_params, &d_token, &pos, &epoch, &d_next, &d_logits};
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
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
