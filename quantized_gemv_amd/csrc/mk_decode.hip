// gfx950 persistent batch-1 decode kernel.
//
// One launch computes one greedy decode step of a Qwen3-style decoder (the
// model of the monolith project page, "Upstream facts"): embedding lookup,
// then per layer RMSNorm -> fused QKV GEMV -> q/k RMSNorm + RoPE + KV append
// -> GQA attention -> O-projection + residual -> RMSNorm -> gate/up GEMV +
// SwiGLU -> down GEMV + residual, then the final RMSNorm, the tied LM-head
// GEMV and the argmax, so one launch yields one token (the page's "fold the LM
// head and argmax into the megakernel").
//
// Launch: one workgroup of eight waves per compute unit, as a plain launch
// once the occupancy check has shown that the device holds the whole grid at
// once (a cooperative launch otherwise).  Wave 0
// of every workgroup is its courier (mk_sync.h): it gathers each input
// vector the workgroup needs from the exchange words, normalises it where the
// consumer wants that (every workgroup recomputes the RMSNorm factor itself,
// the page's trick, so no phase waits for a reduction), and hands it over in
// LDS.  Waves 1..7 compute.  A host-built table gives each compute wave its
// rows of every matrix; the wave keeps those rows' weights in registers and
// loads the next layer's rows of a matrix right after it has used this
// layer's, so about one layer of weights per compute unit is always in
// flight and weight streaming never waits for the dependency chain.
// Attention runs on dedicated workgroups, one per KV head, placed on the XCD
// whose workgroups compute that head's q/k/v rows; each keeps the cached K/V
// rows of its head in registers, loaded one layer ahead.
//
// Weights are dequantized in registers (FP8 and FP4 through the gfx950
// converters) and every product accumulates in fp32 (the page's W8A16
// scheme; the pages' contract also asks for each weight byte to be read once
// per token).  No MFMA: these are matrix-vector products, bound by HBM
// bandwidth.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <stdint.h>

#include "mk.h"
#include "mk_codec.h"
#include "mk_launch.h"
#include "mk_shared.h"
#include "mk_sync.h"
#include "mk_xray.h"

namespace mk {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));

// This wave's index, as a value the compiler knows is uniform across the wave.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Cross-lane reductions with DPP (row operations on the VALU), gfx950's
// permlane swaps and v_readlane.  DPP controls (gfx9): quad_perm [1,0,3,2] =
// 0xB1, [2,3,0,1] = 0x4E, [2,3,2,3] = 0xEE, row_ror:4 = 0x124, row_ror:8 =
// 0x128, row_mirror = 0x140, row_half_mirror = 0x141.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over each 16-lane row, the same bits in every lane of it: each step
// adds a lane's value to its partner's, the partner's partner being the
// lane itself (xor 1, xor 2, then the mirror images within 8 and 16 lanes),
// and a + b == b + a.
__device__ __forceinline__ float sum16(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  return v + dpp<0x140>(v);
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  return fmaxf(v, dpp<0x128>(v));
}
// Sum of a lane's value with those of the lanes 16, 32 and 48 apart (the
// same position in the other 16-lane rows), the same bits in all four:
// v_permlane32_swap pairs lanes 32 apart, v_permlane16_swap rows 16 apart.
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float w = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(w), __float_as_uint(w), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// Sum over the wave, the same bits in every lane (fixed order).
__device__ __forceinline__ float wave_sum(float v) { return rows_sum(sum16(v)); }
// Integer sum over the wave, in every lane: the steps of sum16 and
// rows_sum (exact in any order).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u32<0xB1>(v);
  v += dpp_u32<0x4E>(v);
  v += dpp_u32<0x141>(v);
  v += dpp_u32<0x140>(v);
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = a[0] + a[1];
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return b[0] + b[1];
}
__device__ __forceinline__ float wave_max(float v) {
  v = max16(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
// The row whose total wave_sum4 leaves in lane l: 2 (l & 1) + ((l >> 1) & 1).
__device__ __forceinline__ int sum4_row(int lane) { return 2 * (lane & 1) + ((lane >> 1) & 1); }
// Wave sums of four values at once: lane l ends with the total of value
// sum4_row(l) (lanes 0..3 hold rows 0, 2, 1, 3).  The first two steps
// halve the values per lane while pairing lanes (a lane keeps the rows it
// does not send), the rest sum lanes of the same row: about the cost of one
// full reduction instead of four.  The totals are complete in every lane
// of a row but may differ between its lanes in the last bits (the 16-lane
// steps rotate); callers read one lane per row.
__device__ __forceinline__ float wave_sum4(float a, float b, float c, float d) {
  const int lane = lane_id();
  const bool odd = (lane & 1) != 0, hi = (lane & 2) != 0;
  const float n0 = (odd ? c : a) + dpp<0xB1>(odd ? a : c);   // rows 0 (even lanes), 2 (odd)
  const float n1 = (odd ? d : b) + dpp<0xB1>(odd ? b : d);   // rows 1, 3
  float v = (hi ? n1 : n0) + dpp<0x4E>(hi ? n0 : n1);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  return rows_sum(v);
}

// z * sigmoid(z) with v_exp_f32 and v_rcp_f32 (each within 1 ulp); large
// |z| give z or -0 (exp2 overflows to inf, whose reciprocal is 0).
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// ------------------------------------------------------------------ LDS
// LM-head balancing across XCDs (several steps per launch): grids of up to
// this many workgroups.
constexpr int kLmGrid = 256;

template <int HD, int GS, int NH, int NQ, int NI>
struct Smem {
  // every array starts on a 16-byte boundary: the compute waves read them
  // with 16-byte LDS loads
  alignas(16) float xd_raw[NH * 1024];   // residual entering the layer (fp32)
  alignas(16) uint32_t xd_act[NH * 512]; // its RMSNorm with the layer's input gains, bf16 pairs (QKV input)
  alignas(16) uint32_t o_in[NQ * 512];   // attention output, bf16 pairs (O input)
  alignas(16) float xo_raw[NH * 1024];   // residual after O (fp32)
  alignas(16) uint32_t xo_act[NH * 512]; // its RMSNorm with the post-attention gains (gate/up input)
  alignas(16) uint32_t h_in[NI * 512];   // SwiGLU output, bf16 pairs (down input)
  // attention workgroups
  alignas(16) float qraw[(GS + 2) * HD]; // gathered q heads, k, v of the KV head
  alignas(16) float q[GS * HD];          // normed, roped, pre-scaled q heads
  alignas(16) float kf[HD];              // roped k before rounding
  alignas(16) uint32_t kp[HD / 2];       // this position's k, bf16 pairs
  alignas(16) uint32_t vp[HD / 2];       // this position's v, bf16 pairs
  alignas(16) uint16_t qa[4 * GS][HD];   // q heads as bf16 parts (per head: hi, mid, lo, 0): the score operand
  alignas(16) float part[kCW][GS * HD];  // per wave: unnormalised outputs
  alignas(16) float wm[kCW][GS];         // per wave: running max (log2 units)
  alignas(16) float wl[kCW][GS];         // per wave: running sum
  alignas(16) float sp[GS];              // this position's scores (log2 units)
  alignas(16) float gq[HD], gk[HD];      // q/k-norm gains of the layer
  alignas(16) float rc[HD / 2], rs[HD / 2];   // this position's RoPE cos, sin
  // split attention, home workgroup: the helpers' partials (outputs, then the
  // per-head maxima and sums)
  alignas(16) float spart[kMaxSplit][GS * HD + 2 * GS];
  // argmax
  alignas(16) float best[kCW];
  alignas(16) int32_t bidx[kCW];
  uint32_t seq;                          // inputs handed over by the courier (kAbort: abort)
  uint32_t fail;                         // a wave's step failed: the launch's later steps do not run
  // the launch's step state, read from here by every step (held in no
  // register across a step): step index, steps, first position, first
  // epoch, the next token, and the output arrays' addresses
  uint32_t st_i, st_n, st_pos0, st_e0, st_token;
  uint32_t st_next[2], st_logits[2];
  int tab[kWaves * kSchedInts];          // this workgroup's row of the work table
  uint32_t lm_va, lm_vb;                 // this workgroup's LM-head rows [lm_va, lm_vb) in the step
  uint32_t lm_rec[kLmGrid][2];           // the step before's records: LM-head end tick, dt << 16 | rows << 4 | XCD
  uint32_t arr[kCW];                     // grid-barrier variant: barriers each compute wave has finished its part of
  XR_FIELD
};

// ------------------------------------------------------------------ GEMV
// Lane l covers elements [c*1024 + 16 l, +16) of a row for chunk c, so a
// wave streams each row as contiguous 2 KB (bf16) / 1 KB (fp8) / 512 B (fp4)
// runs with 16-byte (fp4: 8-byte) loads.

// Weights are read through a buffer resource over the arena.  An absent
// unit reads at kOOB (zeros, no memory traffic), so every wave issues the
// same loads in the same order (the compiler's wait counts stay exact) and
// the results are never used.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

struct GMat {
  uint32_t codes, scales, ts;       // byte offsets in the arena
  uint32_t K, ts_mode, ts_b0, ts_b1;
};

__device__ __forceinline__ GMat gmat(const Mat& m, uint64_t off) {
  GMat g;
  g.codes = (uint32_t)(m.codes + off);
  g.scales = (uint32_t)(m.scales + off);
  g.ts = (uint32_t)(m.tscale + off);
  g.K = m.K;
  g.ts_mode = m.ts_mode;
  g.ts_b0 = m.ts_b0;
  g.ts_b1 = m.ts_b1;
  return g;
}

template <uint32_t FMT, int NCH>
struct WRow {
  v4u a[NCH];   // bf16: bytes 0..15 of the lane's 32; fp8: 16 bytes; fp4: 8 bytes of codes in .xy
  v4u b[NCH];   // bf16: bytes 16..31; fp4: the 16-block's E4M3 scale in .x
  float s;      // fp8 row scale / fp4 tensor scale
};

// Load one row's per-lane weights (row < 0: an absent unit, zeros).
template <uint32_t FMT, int NCH>
__device__ __forceinline__ void wrow_load(__amdgpu_buffer_rsrc_t rw, const GMat& g, int row, WRow<FMT, NCH>& w) {
  const int lane = lane_id();
  const bool have = row >= 0;
  const uint32_t r = have ? (uint32_t)row : 0u;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t e0 = (uint32_t)min(c * 1024 + 16 * lane, (int)g.K - 16);
    const uint32_t el = r * g.K + e0;
    if (FMT == FMT_BF16) {
      const uint32_t o = have ? g.codes + 2 * el : kOOB;
      w.a[c] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rw, o, 0, 0));
      w.b[c] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rw, o + 16, 0, 0));
    } else if (FMT == FMT_FP8) {
      w.a[c] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rw, have ? g.codes + el : kOOB, 0, 0));
    } else {
      const v2u c2 = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rw, have ? g.codes + el / 2 : kOOB, 0, 0));
      w.a[c].x = c2.x;
      w.a[c].y = c2.y;
      w.b[c].x = __builtin_amdgcn_raw_buffer_load_b8(rw, have ? g.scales + el / 16 : kOOB, 0, 0);
    }
  }
  if (FMT == FMT_FP8)
    w.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, have ? g.scales + 4 * r : kOOB, 0, 0));
  if (FMT == FMT_FP4) {
    uint32_t idx = 0;
    if (g.ts_mode == 1) idx = r < g.ts_b0 ? 0u : (r < g.ts_b1 ? 1u : 2u);
    else if (g.ts_mode == 2) idx = r & 1u;
    w.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, have ? g.ts + 4 * idx : kOOB, 0, 0));
  }
}

// The lane's part of one row's dot product with the activations xa.
template <uint32_t FMT, int NCH>
__device__ __forceinline__ float wrow_partial(const WRow<FMT, NCH>& w, const uint32_t (&xa)[NCH][8]) {
  float a = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t* xs = xa[c];
    float ac = 0.f;
    if (FMT == FMT_BF16) {
      const uint32_t ws[8] = {w.a[c].x, w.a[c].y, w.a[c].z, w.a[c].w, w.b[c].x, w.b[c].y, w.b[c].z, w.b[c].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) ac = dot2(ws[j], xs[j], ac);
    } else if (FMT == FMT_FP8) {
      const uint32_t ws[4] = {w.a[c].x, w.a[c].y, w.a[c].z, w.a[c].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ac = dot2(e4m3x2_to_bf16x2<false>(ws[j]), xs[2 * j], ac);
        ac = dot2(e4m3x2_to_bf16x2<true>(ws[j]), xs[2 * j + 1], ac);
      }
    } else {
      const uint32_t ws[2] = {w.a[c].x, w.a[c].y};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        ac = dot2(e2m1x2_to_bf16x2<0>(ws[j]), xs[4 * j + 0], ac);
        ac = dot2(e2m1x2_to_bf16x2<1>(ws[j]), xs[4 * j + 1], ac);
        ac = dot2(e2m1x2_to_bf16x2<2>(ws[j]), xs[4 * j + 2], ac);
        ac = dot2(e2m1x2_to_bf16x2<3>(ws[j]), xs[4 * j + 3], ac);
      }
      ac *= e4m3_to_f32(w.b[c].x & 0xFFu);   // the lane's chunk is one 16-block
    }
    a += ac;
  }
  return a;
}

template <uint32_t FMT, int NCH>
__device__ __forceinline__ float wrow_dot(const WRow<FMT, NCH>& w, const uint32_t (&xa)[NCH][8]) {
  float a = wave_sum(wrow_partial(w, xa));
  if (FMT != FMT_BF16) a *= w.s;
  return a;
}

// The lane's activations (bf16 pairs) of a K-element input held in LDS:
// pairs [512 c + 8 l, +8); lanes past K read zeros.
template <int NCH>
__device__ __forceinline__ void load_act(const uint32_t* src, int K, uint32_t (&xa)[NCH][8]) {
  const int lane = lane_id();
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e0 = c * 1024 + 16 * lane;
    const bool in = e0 < K;
    const v4u* xp = reinterpret_cast<const v4u*>(src + min(e0, K - 16) / 2);
    const v4u w0 = xp[0], w1 = xp[1];
    xa[c][0] = in ? w0.x : 0u; xa[c][1] = in ? w0.y : 0u; xa[c][2] = in ? w0.z : 0u; xa[c][3] = in ? w0.w : 0u;
    xa[c][4] = in ? w1.x : 0u; xa[c][5] = in ? w1.y : 0u; xa[c][6] = in ? w1.z : 0u; xa[c][7] = in ? w1.w : 0u;
  }
}

// ------------------------------------------------------------- courier
// A residual vector for LDS and its RMSNorm: pairs j = l + 64k of x (fp32
// bits in lo/hi) go to x_raw (for the residual add after the next
// projection) and bf16(g * (x * r)), r = 1/sqrt(mean(x^2) + eps), to act as
// bf16 pairs in the same order (the GEMVs' input); g[2k], g[2k+1] hold the
// gains of pair j.  The courier does this once for the workgroup, so the
// compute waves only load act.  x_raw holds 128 * MAXK floats and act
// 64 * MAXK pairs: lanes past H/2 store their (don't-care) pairs beyond
// element H, where nobody reads, and add zeros to the sum of squares.
// inv_h = 1/H (exact for a power of two); the reciprocal square root is
// v_rsq_f32 (within 1 ulp).
template <int MAXK>
__device__ __forceinline__ void norm_to_lds(const uint32_t (&lo)[MAXK], const uint32_t (&hi)[MAXK],
                                            const float (&g)[2 * MAXK], int H, float inv_h, float eps,
                                            float* x_raw, uint32_t* act) {
  const int lane = lane_id();
  // four partial sums (pairs k mod 4), added in a fixed order: a quarter of
  // the dependent chain
  float sp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    const bool in = H == 128 * MAXK || lane + 64 * k < H / 2;   // the first: every pair in the vector
    const float a = in ? __uint_as_float(lo[k]) : 0.f, b = in ? __uint_as_float(hi[k]) : 0.f;
    sp[k & 3] = fmaf(a, a, sp[k & 3]);
    sp[k & 3] = fmaf(b, b, sp[k & 3]);
  }
  const float ss = (sp[0] + sp[1]) + (sp[2] + sp[3]);
#pragma unroll
  for (int k = 0; k < MAXK; ++k) *reinterpret_cast<v2u*>(x_raw + 2 * (lane + 64 * k)) = v2u{lo[k], hi[k]};
  const float r = __builtin_amdgcn_rsqf(wave_sum(ss) * inv_h + eps);
#pragma unroll
  for (int k = 0; k < MAXK; ++k)
    act[lane + 64 * k] = pack_bf16(g[2 * k] * (__uint_as_float(lo[k]) * r), g[2 * k + 1] * (__uint_as_float(hi[k]) * r));
}

// The gains of the courier's pairs j = l + 64k of a norm whose bf16
// weights sit at byte `off` of the arena, as fp32 (pairs past H/2 repeat
// the last).  Loaded ahead of the hand-off they serve, so the conversion
// stays off its path.
template <int MAXK>
__device__ __forceinline__ void courier_gains(MK_GLOBAL const uint8_t* W, uint64_t off, int H, float (&g)[2 * MAXK]) {
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    const uint32_t w = GCAST(const uint32_t, W + off)[min(lane_id() + 64 * k, H / 2 - 1)];
    g[2 * k] = bf16_lo(w);
    g[2 * k + 1] = bf16_hi(w);
  }
}

// LONG: the split-attention variant (for long contexts): every GEMV
// workgroup on a KV head's XCD also takes a slice of that head's cached
// positions, and the head's home workgroup merges the slices.
// BAR: the grid-barrier variant, the page's baseline synchronisation kept
// for comparison: every hand-off between phases is one grid-wide barrier
// (each workgroup arrives once its compute waves' stores of the phase are
// complete, with an agent-scope release; all wait for the last arrival, then
// an agent-scope acquire) before any consumer reads the phase's outputs.
// The tagged words are still read after it, so the values are the same
// either way; only the waiting differs.  Not combined with LONG.
template <int WF, int HD, int GS, int NH, int NQ, int NI, bool LONG, bool BAR>
struct Kern {
  static constexpr uint32_t F_LIN = WF == 0 ? FMT_BF16 : (WF == 1 ? FMT_FP8 : FMT_FP4);  // q, k, v, o, gate, up
  static constexpr uint32_t F_8 = WF == 0 ? FMT_BF16 : FMT_FP8;                          // down, embed / LM head
  static constexpr int KX = NH * 8;            // courier pairs per lane: residual vectors
  static constexpr int KO = NQ * 4;            // attention output (bf16 pairs)
  static constexpr int KH = NI * 4;            // SwiGLU output (bf16 pairs)
  static constexpr int KA = ((GS + 2) * HD / 2 + 63) / 64;   // q/k/v of one KV head
  static constexpr int KG = 16;                // argmax words of up to 1024 workgroups
  static constexpr int KL = kLmGrid / 64;      // LM-head balancing: records per lane
  static constexpr int NOUT = GS * HD;         // outputs of one attention workgroup
  static constexpr int PP = (NOUT + 2 * GS) / 2;   // word pairs of one helper partial
  static constexpr int KP = kSplitGatherK;     // helper-partial pairs per lane and round of the home's gather
  static_assert(NOUT <= kCW * 64, "one merge thread per attention output");
  static_assert(!(LONG && BAR), "the grid-barrier variant has no split attention");
  typedef Smem<HD, GS, NH, NQ, NI> S;

  // ------------------------------------------------- grid-barrier variant
  // Barriers of one step, in order: per layer l, 5l + {0: q/k/v, 1: attention
  // output, 2: residual after O, 3: SwiGLU output, 4: residual after down};
  // then 5L: the argmax words.  A compute wave records in s.arr[cw] how many
  // barriers it has finished its part of: after its stores of a phase
  // (in this variant waited for with vmcnt(0), which on gfx9 also waits for
  // its loads in flight), or at once for a phase in which it stores nothing.
  // The tagged exchange keeps the same record, without the wait: there it
  // says that the wave has issued its stores (see stores_out).
  static __device__ __forceinline__ void arrive(S& s, int cw, uint32_t upto, bool stored) {
    if (BAR && stored) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores are complete
    asm volatile("" ::: "memory");
    if (lane_id() == 0) lds_st(&s.arr[cw], upto);
  }

  // Courier, tagged exchange: before polling for the vector of barrier b,
  // wait until this workgroup's compute waves have issued their stores of
  // that phase.  The compute unit's vector-memory path is shared by its
  // waves in issue order, so polls issued earlier would sit ahead of the
  // very stores other workgroups are waiting for; and a vector cannot be
  // complete before this workgroup's part of it is out.  Bounded like every
  // other wait.
  static __device__ __forceinline__ bool stores_out(const Params& p, S& s, uint32_t b) {
    if (BAR) return true;   // the grid barrier before the gather has waited for them
    const int lane = lane_id();
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (true) {
      const uint32_t a = lane < kCW ? lds_ld(&s.arr[lane]) : 0xFFFFFFFFu;
      if (__builtin_amdgcn_ballot_w64(a < b + 1) == 0) return true;
      if (__builtin_amdgcn_s_memrealtime() - t0 > p.spin_limit) {
        raise_error(p, ERR_TIMEOUT);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }

  // Courier: barrier b.  Wait until this workgroup's compute waves have
  // finished their part, then arrive at the grid-wide counter of barrier b
  // and wait until every workgroup of this launch has arrived (the counter
  // reaches the next multiple of the grid).  With p.bar_fence the arrival is
  // an agent-scope release and the departure an agent-scope acquire (on
  // gfx950 an L2 write-back and an L2 invalidate of the workgroup's XCD);
  // without, the counter operations are relaxed agent-scope atomics: the
  // values themselves travel in device-coherent words whose stores the
  // producing waves have waited for.  Bounded like every other wait.
  static __device__ bool grid_barrier(const Params& p, S& s, uint32_t b) {
    const int lane = lane_id();
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (true) {
      const uint32_t a = lane < kCW ? lds_ld(&s.arr[lane]) : 0xFFFFFFFFu;
      if (__builtin_amdgcn_ballot_w64(a < b + 1) == 0) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > p.spin_limit) {
        raise_error(p, ERR_TIMEOUT);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    MK_GLOBAL uint64_t* ctr = p.xch + p.x.bar + b;
    uint64_t old = 0;
    if (lane == 0) {
      if (p.bar_fence)
        old = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      else
        old = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    old = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(old >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)old);
    const uint64_t G = (uint64_t)p.grid, target = (old / G + 1) * G;
    for (uint32_t n = 1;; ++n) {
      const uint64_t v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__builtin_amdgcn_ballot_w64(v < target) == 0) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > p.spin_limit) {
        raise_error(p, ERR_TIMEOUT);
        return false;
      }
      if ((n & 63u) == 0 && __hip_atomic_load(err_word(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
        return false;
      __builtin_amdgcn_s_sleep(1);
    }
    if (p.bar_fence) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
  }

  // ------------------------------------------------------------ courier
  // The inputs this workgroup needs, in order, for every layer; then the
  // final residual for the LM head; workgroup 0 then reduces the argmax.
  // all_argmax: every workgroup reduces the argmax (its result is the next
  // step's token), not only workgroup 0, which writes *d_next.
  // rebalance: a step before this one ran in the launch; the LM-head rows
  // of this step follow from its records (lm_partition).
  static __device__ __forceinline__ bool courier(const Params& p, S& s, const int* hdr, int token, int pos, int ns,
                                 uint32_t epoch, int32_t* d_next, bool all_argmax, bool rebalance,
                                 int& next_token) {
    MK_GLOBAL const uint8_t* const W = p.w;
    const int lane = lane_id();
    const int H = p.H, L = p.L;
    const int flags = hdr[S_FLAGS], att = hdr[S_ATT];
    const __amdgpu_buffer_rsrc_t rs = xch_rsrc(p);
    const Layer& L0 = p.layer0;
    uint32_t seq = 0;
    uint32_t lo[KX], hi[KX];
    const float eps = p.eps, inv_h = 1.0f / (float)H;
    // the lane's input-norm and post-attention-norm gains of the current
    // layer, loaded at the top of the layer (the loads land while the
    // courier waits for this workgroup's stores)
    float gq[2 * KX], gg[2 * KX];
    // where the lane's pairs of the per-producer vectors sit (the same in
    // every layer); its loads go out first, ahead of the embedding's
    uint32_t qm[KA];
    qkv_map(p, att >= 0 ? att : (LONG && hdr[S_SPLIT] >= 0 ? hdr[S_SPLIT] : 0),
            att >= 0 ? (GS + 2) * HD / 2 : NOUT / 2, qm);
    if (flags & 1) courier_gains<KX>(W, p.layer0.in_norm, H, gq);
    // ---- embedding -> the residual of layer 0
    if (flags & 1) {
      XR_PUT(s, 1, XR_START);
#pragma unroll
      for (int k = 0; k < KX; ++k) {
        const int j = min(lane + 64 * k, H / 2 - 1);
        const uint64_t e = (uint64_t)token * H + 2 * j;
        if (F_8 == FMT_BF16) {
          const uint32_t w = *GCAST(const uint32_t, W + p.embed.codes + 2 * e);
          lo[k] = __float_as_uint(bf16_lo(w));
          hi[k] = __float_as_uint(bf16_hi(w));
        } else {
          const uint32_t w = *GCAST(const uint16_t, W + p.embed.codes + e);
          const float sc = GCAST(const float, W + p.embed.scales)[token];
          lo[k] = __float_as_uint(e4m3_to_f32(w & 0xFFu) * sc);
          hi[k] = __float_as_uint(e4m3_to_f32(w >> 8) * sc);
        }
      }
      norm_to_lds<KX>(lo, hi, gq, H, inv_h, eps, s.xd_raw, s.xd_act);
      hand_over(&s.seq, ++seq);
      XR_PUT(s, 1, XR_HANDOFF);
    }
    uint32_t mx[KX], mo[KX], mh[KH];
#pragma unroll
    for (int k = 0; k < KX; ++k) {
      const uint32_t j = (uint32_t)min(lane + 64 * k, H / 2 - 1);
      mx[k] = xpad_word(2 * j, H, p.x.pad_c[V_XD], p.x.pad_stride[V_XD]);
      mo[k] = xpad_word(2 * j, H, p.x.pad_c[V_XO], p.x.pad_stride[V_XO]);
    }
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      const uint32_t j = (uint32_t)min(lane + 64 * k, p.I / 4 - 1);
      mh[k] = xpad_word(2 * j, p.I / 2, p.x.pad_c[V_H], p.x.pad_stride[V_H]);
    }
    // attention and split-attention helper workgroups: layer 0's q/k-norm
    // gains and the position's RoPE pair (the same in every layer)
    const bool att_in = att >= 0 || (LONG && hdr[S_SPLIT] >= 0);
    uint32_t ag[4] = {0u, 0u, 0u, 0u};
    float rc = 0.f, rsn = 0.f;
    if (att_in) {
      att_gains(p, 0, ag);
      MK_GLOBAL const float* cs = p.rope + ((size_t)pos * (HD / 2) + min(lane, HD / 2 - 1)) * 2;
      rc = cs[0];
      rsn = cs[1];
    }
    // this step's LM-head rows: a GEMV workgroup's courier now (the compute
    // waves' layer-0 QKV rows cover it), an attention workgroup's after its
    // layer-0 attention, where it waits for the next layer's q, k, v
    XR_PUT(s, 1, XR_M0);
    if (rebalance && att < 0) lm_partition(p, s);
    XR_PUT(s, 1, XR_M0 + 1);
    for (int l = 0; l < L; ++l) {
      const uint64_t loff = (uint64_t)l * p.layer_stride;
      const int ph = 2 + 6 * l;
      const uint32_t bq = 5u * (uint32_t)l;
      if ((flags & 1) && l > 0) courier_gains<KX>(W, p.layer0.in_norm + loff, H, gq);
      if (flags & 4) courier_gains<KX>(W, p.layer0.post_norm + loff, H, gg);
      // ---- residual entering layer l (layer 0: the embedding above)
      if (BAR && l > 0 && !grid_barrier(p, s, bq - 1)) return abort(s);
      if ((flags & 1) && l > 0) {
        if (!stores_out(p, s, bq - 1)) return abort(s);
        XR_PUT(s, ph + 0, XR_START);
        if (!gather_pairs_at<KX>(p, rs, H / 2, make_tag(epoch, vec_id(l - 1, V_XD)), lo, hi, xword(p, l - 1, V_XD),
                                 mx))
          return abort(s);
        XR_PUT(s, ph + 0, XR_READY);
        norm_to_lds<KX>(lo, hi, gq, H, inv_h, eps, s.xd_raw, s.xd_act);
        hand_over(&s.seq, ++seq);
        XR_PUT(s, ph + 0, XR_HANDOFF);
      }
      if (att < 0) lds_barrier();   // the compute waves' QKV stores are out; their weight burst follows
      if (BAR && !grid_barrier(p, s, bq + 0)) return abort(s);
      // ---- q, k, v of KV head `att`: q/k RMSNorm, RoPE, KV append
      if (att >= 0) {
        XR_PUT(s, ph + 1, XR_START);
        if (!attention_input<true>(p, s, l, att, pos, epoch, rs, qm, ag, rc, rsn)) return abort(s);
        hand_over(&s.seq, ++seq);
        XR_PUT(s, ph + 1, XR_HANDOFF);
        lds_barrier();   // q, k and v are normed, roped and appended
        lds_barrier();   // every compute wave has written its partial outputs
        if (LONG && ns > 0) lds_barrier();   // the helpers' partials are in LDS
        lds_barrier();   // and merged them: the LDS arrays may be reused
        if (l == 0 && rebalance) lm_partition(p, s);
      }
      // ---- split attention helper: q of KV head hdr[S_SPLIT]
      if (LONG && hdr[S_SPLIT] >= 0) {
        if (hdr[S_SPLIT_IDX] <= ns) {
          XR_PUT(s, ph + 1, XR_START);
          if (!attention_input<false>(p, s, l, hdr[S_SPLIT], pos, epoch, rs, qm, ag, rc, rsn)) return abort(s);
          hand_over(&s.seq, ++seq);
          XR_PUT(s, ph + 1, XR_HANDOFF);
          lds_barrier();   // q is normed and roped
          lds_barrier();   // every compute wave has written its partial outputs
        } else {
          hand_over(&s.seq, ++seq);   // no slice this step; keeps the input numbering
        }
      }
      // the next layer's gains, while the courier waits for its q, k, v
      if (att_in) att_gains(p, min(l + 1, L - 1), ag);
      // ---- attention output
      if (BAR && !grid_barrier(p, s, bq + 1)) return abort(s);
      if (flags & 2) {
        XR_PUT(s, ph + 3, XR_START);
        uint32_t ol[KO], oh[KO];
        const uint32_t base = (uint32_t)(xvec(p, l, V_O) - p.xch);
        if (!gather_pairs<KO>(p, rs, p.nq * HD / 4, make_tag(epoch, vec_id(l, V_O)), ol, oh,
                              [=](int j) { return base + 2u * j; }))
          return abort(s);
        XR_PUT(s, ph + 3, XR_READY);
#pragma unroll
        for (int k = 0; k < KO; ++k)   // o_in holds 64 * KO pairs: lanes past the end store don't-care pairs there
          *reinterpret_cast<v2u*>(s.o_in + 2 * (lane + 64 * k)) = v2u{ol[k], oh[k]};
        hand_over(&s.seq, ++seq);
        XR_PUT(s, ph + 3, XR_HANDOFF);
      }
      // ---- residual after O
      if (BAR && !grid_barrier(p, s, bq + 2)) return abort(s);
      if (flags & 4) {
        if (!stores_out(p, s, bq + 2)) return abort(s);
        XR_PUT(s, ph + 4, XR_START);
        if (!gather_pairs_at<KX>(p, rs, H / 2, make_tag(epoch, vec_id(l, V_XO)), lo, hi, xword(p, l, V_XO), mo))
          return abort(s);
        XR_PUT(s, ph + 4, XR_READY);
        norm_to_lds<KX>(lo, hi, gg, H, inv_h, eps, s.xo_raw, s.xo_act);
        hand_over(&s.seq, ++seq);
        XR_PUT(s, ph + 4, XR_HANDOFF);
      }
      // ---- SwiGLU output
      if (BAR && !grid_barrier(p, s, bq + 3)) return abort(s);
      if (flags & 8) {
        if (!stores_out(p, s, bq + 3)) return abort(s);
        XR_PUT(s, ph + 5, XR_START);
        uint32_t hl[KH], hh[KH];
        if (!gather_pairs_at<KH>(p, rs, p.I / 4, make_tag(epoch, vec_id(l, V_H)), hl, hh, xword(p, l, V_H), mh))
          return abort(s);
        XR_PUT(s, ph + 5, XR_READY);
#pragma unroll
        for (int k = 0; k < KH; ++k)   // h_in holds 64 * KH pairs: lanes past the end store don't-care pairs there
          *reinterpret_cast<v2u*>(s.h_in + 2 * (lane + 64 * k)) = v2u{hl[k], hh[k]};
        hand_over(&s.seq, ++seq);
        XR_PUT(s, ph + 5, XR_HANDOFF);
      }
    }
    // ---- final residual -> final RMSNorm (LM-head input)
    const int ph_head = 2 + 6 * L;
    if (BAR && !grid_barrier(p, s, 5u * (uint32_t)L - 1u)) return abort(s);
    {
      courier_gains<KX>(W, p.final_norm, H, gq);
      if (!stores_out(p, s, 5u * (uint32_t)L - 1u)) return abort(s);
      XR_PUT(s, ph_head, XR_START);
      if (!gather_pairs_at<KX>(p, rs, H / 2, make_tag(epoch, vec_id(L - 1, V_XD)), lo, hi, xword(p, L - 1, V_XD),
                               mx))
        return abort(s);
      XR_PUT(s, ph_head, XR_READY);
      norm_to_lds<KX>(lo, hi, gq, H, inv_h, eps, s.xd_raw, s.xd_act);
      hand_over(&s.seq, ++seq);
      XR_PUT(s, ph_head, XR_HANDOFF);
    }
    lds_barrier();   // the compute waves' argmax candidates are in LDS
    if (BAR && !grid_barrier(p, s, 5u * (uint32_t)L)) return false;
    // ---- workgroup 0 (every workgroup when a step follows in this launch):
    // reduce every workgroup's (value, index)
    if (blockIdx.x == 0 || all_argmax) {
      XR_PUT(s, ph_head + 1, XR_START);
      const uint32_t base = (uint32_t)p.x.arg;
      const uint32_t tag = make_tag(epoch, vec_id(L, 0));
      float best = -INFINITY;
      int bidx = 0x7FFFFFFF;
      auto take = [&](uint32_t vw, uint32_t iw) {
        const float v = __uint_as_float(vw);
        const int i = (int)iw;
        if (v > best || (v == best && i < bidx)) {
          best = v;
          bidx = i;
        }
      };
      if (all_argmax && p.lm_balance && p.grid <= kLmGrid) {
        // whole records, one round: pair 2j is workgroup j's (value, index),
        // pair 2j + 1 its (end tick, dt << 16 | rows << 4 | XCD), kept for the
        // next step's LM-head rows (even lanes hold the former, odd lanes the
        // latter)
        uint32_t al[2 * KL], ah[2 * KL];
        if (!gather_pairs<2 * KL>(p, rs, 2 * p.grid, tag, al, ah, [=](int j) { return base + 2u * j; }))
          return false;
        XR_PUT(s, ph_head + 1, XR_READY);
#pragma unroll
        for (int k = 0; k < 2 * KL; ++k) {
          const int j = lane + 64 * k;
          if (j < 2 * p.grid) {
            if ((lane & 1) == 0) {
              take(al[k], ah[k]);
            } else {
              s.lm_rec[j >> 1][0] = al[k];
              s.lm_rec[j >> 1][1] = ah[k];
            }
          }
        }
      } else if (p.grid <= kLmGrid) {
        // the (value, index) pairs alone: KL loads per lane
        uint32_t vl[KL], il[KL];
        if (!gather_pairs<KL>(p, rs, p.grid, tag, vl, il, [=](int j) { return base + 4u * j; })) return false;
        XR_PUT(s, ph_head + 1, XR_READY);
#pragma unroll
        for (int k = 0; k < KL; ++k)
          if (lane + 64 * k < p.grid) take(vl[k], il[k]);
      } else {
        uint32_t vl[KG], il[KG];
        if (!gather_pairs<KG>(p, rs, p.grid, tag, vl, il, [=](int j) { return base + 4u * j; })) return false;
        XR_PUT(s, ph_head + 1, XR_READY);
#pragma unroll
        for (int k = 0; k < KG; ++k)
          if (lane + 64 * k < p.grid) take(vl[k], il[k]);
      }
      const float m = wave_max(best);
      int mi = best == m ? bidx : 0x7FFFFFFF;   // smallest index among the lanes holding the maximum
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mi = min(mi, __shfl_xor(mi, o));
      next_token = __builtin_amdgcn_readfirstlane(mi);
      if (blockIdx.x == 0 && lane == 0) *d_next = mi;
      XR_PUT(s, ph_head + 1, XR_HANDOFF);
    }
    return true;
  }

  // This step's LM-head rows, from every workgroup's record of the step
  // before (gathered with the argmax into lm_rec): a damped step towards
  // equal end times.  Each workgroup's share moves by half of its end's
  // offset from the grid's mean end, converted to rows with its own rows per
  // tick (the workgroups of a slower XCD all end later and all give rows
  // away); the rows then go to workgroups in index order in proportion to
  // their shares.  Every workgroup runs the same instructions on the same
  // words, so all of them derive the same partition of [0, V): workgroup w's
  // end and workgroup w+1's start are the same function of the same prefix
  // sum.  Which workgroup computes a row changes neither its logit nor the
  // argmax.  Equal shares when the LM head is too short to time (under a
  // microsecond on average) or a share would not fit the record's 12 bits of
  // rows; grids of up to kLmGrid workgroups.
  static __device__ void lm_partition(const Params& p, S& s) {
    const int lane = lane_id(), G = p.grid, wg = blockIdx.x;
    if (!p.lm_balance || G > kLmGrid || 2 * p.V / G > 0xFFF) return;
    uint32_t te[KL], mt[KL];   // end ticks, dt << 16 | rows << 4 | XCD
    const uint32_t e0 = s.lm_rec[0][0];
    uint32_t es = 0, ds = 0;
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      const int j = lane + 64 * k;
      te[k] = s.lm_rec[min(j, G - 1)][0];
      mt[k] = s.lm_rec[min(j, G - 1)][1];
      es += j < G ? te[k] - e0 : 0u;   // ends past workgroup 0's (two's complement: earlier ones subtract)
      ds += j < G ? mt[k] >> 16 : 0u;
    }
    const float emean = (float)(int)wave_sum_u32(es) / (float)G;
    const bool even = wave_sum_u32(ds) < 100u * (uint32_t)G;   // 100 ticks: 1 us
    uint32_t sw = 0, sw1 = 0, st = 0;   // this lane's share of S(wg), S(wg + 1) and S(G), in 1/16 rows
#pragma unroll
    for (int k = 0; k < KL; ++k) {
      const int j = lane + 64 * k;
      const float r = (float)((mt[k] >> 4) & 0xFFFu);
      const float d = (float)max(mt[k] >> 16, 1u);
      const float e = (float)(int)(te[k] - e0);
      const float w = even ? 1.f : fminf(fmaxf(r - 0.5f * (e - emean) * (r / d), 0.5f * r), 2.f * r);
      const uint32_t wi = j < G ? (uint32_t)(w * 16.f + 0.5f) + 1u : 0u;
      sw += j < wg ? wi : 0u;
      sw1 += j <= wg ? wi : 0u;
      st += wi;
    }
    sw = wave_sum_u32(sw);
    sw1 = wave_sum_u32(sw1);
    st = wave_sum_u32(st);
    const double vs = (double)p.V / (double)st;
    if (lane == 0) {
      lds_st(&s.lm_va, wg == 0 ? 0u : min((uint32_t)((double)sw * vs), (uint32_t)p.V));
      lds_st(&s.lm_vb, wg == G - 1 ? (uint32_t)p.V : min((uint32_t)((double)sw1 * vs), (uint32_t)p.V));
    }
  }

  static __device__ bool abort(S& s) {
    hand_over(&s.seq, kAbort);
    return false;
  }

  // The word offsets (in the q/k/v vector) of the lane's pairs of KV head
  // g's q, k and v rows, from the map in the work table (read once per
  // launch; pairs past the first np repeat the last one).
  static __device__ __forceinline__ void qkv_map(const Params& p, int g, int np, uint32_t (&qm)[KA]) {
    MK_GLOBAL const int* m = GCAST(const int, p.w + p.qmap) + (size_t)g * ((GS + 2) * HD / 2);
#pragma unroll
    for (int k = 0; k < KA; ++k) qm[k] = (uint32_t)m[min(lane_id() + 64 * k, np - 1)];
  }

  // The q/k-norm gains of layer l at this lane's RoPE pair (lane,
  // lane + HD/2), as loaded bf16 bits: the courier loads the next layer's
  // while it waits, and converts them where they are used, so that no wait
  // for them sits in front of the q/k/v gather's first poll round.
  static __device__ __forceinline__ void att_gains(const Params& p, int l, uint32_t (&ag)[4]) {
    const int li = min(lane_id(), HD / 2 - 1);
    const uint64_t loff = (uint64_t)l * p.layer_stride;
    MK_GLOBAL const uint16_t* gq = GCAST(const uint16_t, p.w + p.layer0.q_norm + loff);
    MK_GLOBAL const uint16_t* gk = GCAST(const uint16_t, p.w + p.layer0.k_norm + loff);
    ag[0] = gq[li];
    ag[1] = gq[li + HD / 2];
    ag[2] = gk[li];
    ag[3] = gk[li + HD / 2];
  }

  // Gather q (GS heads), k and v of KV head g into LDS, with this layer's
  // q/k-norm gains and this position's RoPE pairs; the compute waves norm,
  // rope and append them (att_prepare).  Without KV (a split-attention
  // helper): q only, with the q-norm gains.  qm: the word offsets of the
  // lane's pairs (see qkv_map); ag: att_gains(l); rc, rsn: the position's
  // RoPE pair of this lane (loaded by the courier before its layer loop).
  template <bool KV>
  static __device__ bool attention_input(const Params& p, S& s, int l, int g, int pos, uint32_t epoch,
                                         __amdgpu_buffer_rsrc_t rs, const uint32_t (&qm)[KA],
                                         const uint32_t (&ag)[4], float rc, float rsn) {
    const int lane = lane_id();
    constexpr int NP = KV ? (GS + 2) * HD / 2 : NOUT / 2;   // pairs gathered
    constexpr int K = (NP + 63) / 64;
    uint32_t lo[K], hi[K], off[K];
#pragma unroll
    for (int k = 0; k < K; ++k) off[k] = qm[k];
    if (!gather_pairs_at<K>(p, rs, NP, make_tag(epoch, vec_id(l, V_QKV)), lo, hi, xword(p, l, V_QKV), off))
      return false;
    XR_PUT(s, 2 + 6 * l + 1, XR_READY);
    static_assert(NP % 64 == 0, "every lane stores a pair of q/k/v");
#pragma unroll
    for (int k = 0; k < K; ++k) *reinterpret_cast<v2u*>(s.qraw + 2 * (lane + 64 * k)) = v2u{lo[k], hi[k]};
    if (lane < HD / 2) {
      s.gq[lane] = bf16_to_f32((uint16_t)ag[0]);
      s.gq[lane + HD / 2] = bf16_to_f32((uint16_t)ag[1]);
      s.gk[lane] = bf16_to_f32((uint16_t)ag[2]);
      s.gk[lane + HD / 2] = bf16_to_f32((uint16_t)ag[3]);
      s.rc[lane] = rc;
      s.rs[lane] = rsn;
    }
    return true;
  }

  // Compute wave cw of an attention workgroup, once the raw q/k/v are in
  // LDS: waves 0..GS-1 RMSNorm and rope q head cw (pre-scaled by
  // log2(e)/sqrt(HD), so scores come out in log2 units); wave GS does k
  // (rounded to bf16 as the cache holds it) and wave GS+1 rounds v; both
  // append to the cache at `pos`.  Lane i < HD/2 owns the RoPE pair
  // (i, i + HD/2).
  // Without KV (a split-attention helper): the q heads only.
  template <bool KV>
  static __device__ __forceinline__ void att_prepare(const Params& p, S& s, int l, int g, int pos, int cw, bool ok) {
    const int lane = lane_id();
    const bool pl = lane < HD / 2;
    const int li = min(lane, HD / 2 - 1);
    if (cw < GS || (KV && cw == GS)) {
      const float* src = s.qraw + cw * HD;
      const float xa = pl ? src[li] : 0.f, xb = pl ? src[li + HD / 2] : 0.f;
      const float r = __builtin_amdgcn_rsqf(wave_sum(xa * xa + xb * xb) * (1.0f / HD) + p.eps);   // v_rsq_f32: within 1 ulp
      const float* gg = cw < GS ? s.gq : s.gk;
      const float a = gg[li] * (xa * r), b = gg[li + HD / 2] * (xb * r);
      const float c = s.rc[li], sn = s.rs[li];
      const float ra = a * c - b * sn, rb = b * c + a * sn;
      if (cw < GS) {
        const float kq = 1.4426950408889634f / sqrtf((float)HD);
        if (pl) {
          const float qa = ra * kq, qb = rb * kq;
          s.q[cw * HD + li] = qa;
          s.q[cw * HD + li + HD / 2] = qb;
          uint32_t pa[3], pb[3];
          split3(qa, pa);
          split3(qb, pb);
#pragma unroll
          for (int k = 0; k < 3; ++k) {
            s.qa[4 * cw + k][li] = (uint16_t)pa[k];
            s.qa[4 * cw + k][li + HD / 2] = (uint16_t)pb[k];
          }
        }
      } else {
        if (pl) {
          s.kf[li] = ra;
          s.kf[li + HD / 2] = rb;
        }
        lds_drain();
        if (pl) {
          const uint32_t kw = pack_bf16(s.kf[2 * lane], s.kf[2 * lane + 1]);
          s.kp[lane] = kw;
          MK_GLOBAL uint32_t* kc = GCAST(uint32_t, p.kv + ((size_t)(l * 2 + 0) * p.nkv + g) * kv_plane(p));
          if (ok) kc[(size_t)pos * (HD / 2) + lane] = kw;   // an aborted step leaves the cache alone
        }
      }
    } else if (KV && cw == GS + 1) {
      if (pl) {
        const float* vf = s.qraw + (GS + 1) * HD;
        const uint32_t vw = pack_bf16(vf[2 * lane], vf[2 * lane + 1]);
        s.vp[lane] = vw;
        // the V plane is tiled by 4 positions: (j, e) at (j/4 * HD + e) * 4 + j%4
        MK_GLOBAL uint16_t* vc = GCAST(uint16_t, p.kv + ((size_t)(l * 2 + 1) * p.nkv + g) * kv_plane(p));
        const size_t e0 = ((size_t)(pos >> 2) * HD + 2 * lane) * 4 + (pos & 3);
        if (ok) {
          vc[e0] = (uint16_t)vw;
          vc[e0 + 4] = (uint16_t)(vw >> 16);
        }
      }
    }
  }

  // Scores of the current position for every q head (its k as the cache
  // holds it, bf16), into s.sp; one wave, after att_prepare.
  static __device__ __forceinline__ void att_current_scores(S& s) {
    const int lane = lane_id();
    const uint32_t kw = lane < HD / 2 ? s.kp[lane] : 0u;
#pragma unroll
    for (int h = 0; h < GS; ++h) {
      const float d =
          lane < HD / 2 ? s.q[h * HD + 2 * lane] * bf16_lo(kw) + s.q[h * HD + 2 * lane + 1] * bf16_hi(kw) : 0.f;
      const float sc = wave_sum(d);
      if (lane == 0) s.sp[h] = sc;
    }
  }

  // --------------------------------------------------- GEMV compute waves
  // Every branch below depends on wave-uniform values only and holds no
  // global load, and a wave's stores go through buffer offsets (kOOB drops
  // them) instead of branches, so all paths through a layer issue the same
  // vector-memory operations and the compiler's vmcnt waits for each
  // matrix's rows count exactly the loads issued after them.  An abort is
  // not an early exit (that would add a path to the loop latch with fewer
  // loads and make every wait conservative): the remaining phases run on
  // whatever LDS holds and store nothing.
  //
  // Weight loads go out in one burst per layer, right after the wave's QKV
  // rows are published: the O, gate/up and down rows of this layer and the
  // QKV rows of the next (in bf16 those follow the O-projection's stores).  While the attention workgroups work, nothing is
  // exchanged, so the burst drains then; the later exchanges of the layer
  // travel through an idle memory system.  An exchange word that waits
  // behind a full HBM queue takes several microseconds instead of well
  // under one.
  struct GemvW {
    WRow<F_LIN, NH> q[kMaxQKV];
    WRow<F_LIN, NQ> o[kMaxO];
    WRow<F_LIN, NH> gu[kMaxGU][4];
    WRow<F_8, NI> d[kMaxD];
    uint32_t so[kMaxO], sg[kMaxGU], sd[kMaxD];   // output word of each O / gate-up / down unit
  };

  // have = false (past the last layer): the same loads at the offset past
  // the arena (zeros, no memory access), so the last layer runs the same
  // instructions as every other.
  static __device__ __forceinline__ void load_layer_qkv(const Params& p, __amdgpu_buffer_rsrc_t rw, const int* u,
                                                        int l, GemvW& w, bool have = true) {
    const uint64_t lo = (uint64_t)l * p.layer_stride;
    const GMat g = gmat(p.layer0.qkv, lo);
#pragma unroll
    for (int k = 0; k < kMaxQKV; ++k) wrow_load(rw, g, have ? u[S_QKV + k] : -1, w.q[k]);
  }
  static __device__ __forceinline__ void load_layer_o(const Params& p, __amdgpu_buffer_rsrc_t rw, const int* u,
                                                      int l, GemvW& w) {
    const GMat go = gmat(p.layer0.o, (uint64_t)l * p.layer_stride);
#pragma unroll
    for (int k = 0; k < kMaxO; ++k) wrow_load(rw, go, u[S_O + k], w.o[k]);
  }
  static __device__ __forceinline__ void load_layer_mlp(const Params& p, __amdgpu_buffer_rsrc_t rw, const int* u,
                                                        int l, GemvW& w) {
    const uint64_t lo = (uint64_t)l * p.layer_stride;
    const GMat gg = gmat(p.layer0.gu, lo);
#pragma unroll
    for (int k = 0; k < kMaxGU; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) wrow_load(rw, gg, u[S_GU + k] >= 0 ? 4 * u[S_GU + k] + r : -1, w.gu[k][r]);
    const GMat gd = gmat(p.layer0.down, lo);
#pragma unroll
    for (int k = 0; k < kMaxD; ++k) wrow_load(rw, gd, u[S_D + k], w.d[k]);
  }

  // bf16: the next layer's QKV rows are loaded after this layer's
  // O-projection stores instead of in the burst during attention (measured:
  // 0.3 % per token at the 0.6B shape, whose bf16 burst is 30 MB).  FP8 and
  // FP4 keep them in the burst.
  static constexpr bool kQkvLate = F_LIN == FMT_BF16;
  // One layer of a GEMV compute wave; the burst (bf16: the O phase) also
  // loads the next layer's QKV rows (past the last layer: no-op loads).  One
  // instance serves every layer, which keeps the kernel's code within the
  // instruction cache.
  static __device__ __forceinline__ bool gemv_layer(const Params& p, S& s, int l, const int* hdr, const int* u,
                                                    GemvW& w, int pos, int ns, int cw, uint32_t epoch,
                                                    __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx, bool ok) {
    const bool l0 = lane_id() == 0;
    const int H = p.H, nin = LONG ? hdr[S_NIN_L] : hdr[S_NIN];
    const int i_o = LONG ? hdr[S_IO_L] : hdr[S_IO], i_xo = LONG ? hdr[S_IXO_L] : hdr[S_IXO];
    const int i_h = LONG ? hdr[S_IH_L] : hdr[S_IH];
    const uint32_t sbase = (uint32_t)(l * nin) + 1u;
    const int ph = 2 + 6 * l;
    // ---- QKV
    {
      if (u[S_QKV] >= 0) {
        ok = ok && wait_seq(p, &s.seq, sbase + hdr[S_IXD]);
        XR_MIN(s, ph + 0, XR_SEEN);
      }
      if (u[S_QKV] >= 0) {
      uint32_t xa[NH][8];
      load_act<NH>(s.xd_act, H, xa);
#ifdef MK_XRAY
      {  // X-ray: when this wave's QKV rows are all in registers
        uint32_t z = 0;
#pragma unroll
        for (int k = 0; k < kMaxQKV; ++k) z ^= w.q[k].a[NH - 1].w ^ w.q[k].b[NH - 1].w;
        asm volatile("" ::"v"(z));
        if (u[S_QKV] >= 0) XR_MAX(s, ph + 0, XR_M0);
      }
#endif
      const uint32_t base = xword(p, l, V_QKV), tag = make_tag(epoch, vec_id(l, V_QKV));
      static_assert(kMaxQKV <= 4, "one wave_sum4 for the q/k/v rows");
      float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < kMaxQKV; ++k) y[k] = wrow_partial(w.q[k], xa);
      // lane q < kMaxQKV (q = sum4_row(lane), lanes 0..3) stores row q
      const int q = sum4_row(lane_id());
      float v = wave_sum4(y[0], y[1], y[2], y[3]);
      int r = u[S_QKV];
      uint32_t wo = (uint32_t)u[S_QKVW];
      float sc = w.q[0].s;
#pragma unroll
      for (int k = 1; k < kMaxQKV; ++k) {
        r = q == k ? u[S_QKV + k] : r;
        wo = q == k ? (uint32_t)u[S_QKVW + k] : wo;
        sc = q == k ? w.q[k].s : sc;
      }
      if (F_LIN != FMT_BF16) v *= sc;
      st_xword(rx, ok && lane_id() < 4 && q < kMaxQKV && r >= 0 ? 8u * (base + wo) : kOOB, __float_as_uint(v), tag);
      XR_MAX(s, ph + 0, XR_DONE);
      }
    }
    arrive(s, cw, 5u * (uint32_t)l + 2u, true);   // q/k/v stored; nothing of the attention output
    // ---- the layer's weight burst, once every wave of the workgroup has
    // issued its QKV stores (the courier joins this barrier after handing
    // over the layer's input): a burst queued ahead of another wave's stores
    // would delay the attention workgroups' input by the burst's issue time.
    // With split attention a helper's slice runs before the burst, so that
    // it has the registers of the O, gate/up, down and next QKV rows; its
    // first pass of cached rows goes out before the wait for q.
    lds_barrier();
    if (!LONG) {
      load_layer_o(p, rw, u, l, w);
      load_layer_mlp(p, rw, u, l, w);
      if constexpr (!kQkvLate) load_layer_qkv(p, rw, u, l + 1, w, l + 1 < p.L);
    } else {
      // a helper's first pass of cached rows does not depend on this step's q
      const bool help = hdr[S_SPLIT] >= 0 && hdr[S_SPLIT_IDX] <= ns;
      KVBlock k0;
      if (help) help_issue(p, l, hdr[S_SPLIT], hdr[S_SPLIT_IDX], pos, ns, cw, k0);
      if (help)
        ok = att_help(p, s, l, hdr[S_SPLIT], hdr[S_SPLIT_IDX], pos, ns, cw, sbase + hdr[S_IQS_L], epoch, rx, ok, k0);
      load_layer_o(p, rw, u, l, w);
      load_layer_mlp(p, rw, u, l, w);
      load_layer_qkv(p, rw, u, l + 1, w, l + 1 < p.L);
    }
    // ---- O-projection + residual
    {
      if (u[S_O] >= 0) {
        ok = ok && wait_seq(p, &s.seq, sbase + i_o);
        XR_MIN(s, ph + 3, XR_SEEN);
      }
      if (u[S_O] >= 0) {
      uint32_t xa[NQ][8];
      load_act<NQ>(s.o_in, p.nq * HD, xa);
      const uint32_t base = xword(p, l, V_XO), tag = make_tag(epoch, vec_id(l, V_XO));
#pragma unroll
      for (int k = 0; k < kMaxO; ++k) {
        const int r = u[S_O + k];
        const float v = s.xd_raw[max(r, 0)] + wrow_dot(w.o[k], xa);
        st_xword(rx, ok && r >= 0 && l0 ? 8u * (base + w.so[k]) : kOOB, __float_as_uint(v), tag);
      }
      XR_MAX(s, ph + 3, XR_DONE);
      }
    }
    arrive(s, cw, 5u * (uint32_t)l + 3u, true);
    if constexpr (!LONG && kQkvLate) load_layer_qkv(p, rw, u, l + 1, w, l + 1 < p.L);
    // ---- gate/up + SwiGLU: a unit is the four rows behind one output word
    {
      if (u[S_GU] >= 0) {
        ok = ok && wait_seq(p, &s.seq, sbase + i_xo);
        XR_MIN(s, ph + 4, XR_SEEN);
      }
      if (u[S_GU] >= 0) {
      uint32_t xa[NH][8];
      load_act<NH>(s.xo_act, H, xa);
      const uint32_t base = xword(p, l, V_H), tag = make_tag(epoch, vec_id(l, V_H));
#pragma unroll
      for (int k = 0; k < kMaxGU; ++k) {
        const int t = u[S_GU + k];
        if (k > 0 && t < 0) break;   // wave-uniform, and no load inside the loop
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = wrow_partial(w.gu[k][r], xa);
        // rows (gate, up, gate, up): lanes 0, 2, 1, 3 end with their totals
        const int q = sum4_row(lane_id());
        float v = wave_sum4(y[0], y[1], y[2], y[3]);
        if (F_LIN != FMT_BF16)
          v *= q == 0 ? w.gu[k][0].s : (q == 1 ? w.gu[k][1].s : (q == 2 ? w.gu[k][2].s : w.gu[k][3].s));
        const float h = silu(v) * dpp<0xEE>(v);   // lane 0: gate 0 with up 0 (lane 2); lane 1: rows 2, 3
        st_xword(rx, ok && t >= 0 && l0 ? 8u * (base + w.sg[k]) : kOOB, pack_bf16(h, dpp<0xB1>(h)), tag);
      }
      XR_MAX(s, ph + 4, XR_DONE);
      }
    }
    arrive(s, cw, 5u * (uint32_t)l + 4u, true);
    // ---- down + residual
    {
      if (u[S_D] >= 0) {
        ok = ok && wait_seq(p, &s.seq, sbase + i_h);
        XR_MIN(s, ph + 5, XR_SEEN);
      }
      if (u[S_D] >= 0) {
      uint32_t xa[NI][8];
      load_act<NI>(s.h_in, p.I, xa);
      const uint32_t base = xword(p, l, V_XD), tag = make_tag(epoch, vec_id(l, V_XD));
#pragma unroll
      for (int k = 0; k < kMaxD; ++k) {
        const int r = u[S_D + k];
        const float v = s.xo_raw[max(r, 0)] + wrow_dot(w.d[k], xa);
        st_xword(rx, ok && r >= 0 && l0 ? 8u * (base + w.sd[k]) : kOOB, __float_as_uint(v), tag);
      }
      XR_MAX(s, ph + 5, XR_DONE);
      }
    }
    arrive(s, cw, 5u * (uint32_t)l + 5u, true);
    return ok;
  }

  // The output words of the wave's O, gate/up and down units (once per
  // launch).
  static __device__ __forceinline__ void gemv_setup(const Params& p, const int* u, GemvW& w) {
#pragma unroll
    for (int k = 0; k < kMaxO; ++k)
      w.so[k] = xpad_word((uint32_t)max(u[S_O + k], 0), p.H, p.x.pad_c[V_XO], p.x.pad_stride[V_XO]);
#pragma unroll
    for (int k = 0; k < kMaxGU; ++k)
      w.sg[k] = xpad_word((uint32_t)max(u[S_GU + k], 0), p.I / 2, p.x.pad_c[V_H], p.x.pad_stride[V_H]);
#pragma unroll
    for (int k = 0; k < kMaxD; ++k)
      w.sd[k] = xpad_word((uint32_t)max(u[S_D + k], 0), p.H, p.x.pad_c[V_XD], p.x.pad_stride[V_XD]);
  }
  // bf16: layer 0's QKV rows are loaded before the step, during the
  // previous step's argmax when one ran.  In FP8 and FP4 the same early
  // load changed the layer loop's register allocation and cost more than it
  // saved (measured), so there each step loads them itself.
  static constexpr bool kQKV0Early = F_LIN == FMT_BF16;
  // The layers of one step.
  static __device__ __forceinline__ bool gemv_waves(const Params& p, S& s, const int* hdr, const int* u, int pos,
                                                    int ns, int cw, uint32_t epoch, __amdgpu_buffer_rsrc_t rw,
                                                    __amdgpu_buffer_rsrc_t rx, GemvW& w) {
    gemv_setup(p, u, w);
    if constexpr (!kQKV0Early) load_layer_qkv(p, rw, u, 0, w);
    bool ok = true;
    for (int l = 0; l < p.L; ++l) ok = gemv_layer(p, s, l, hdr, u, w, pos, ns, cw, epoch, rw, rx, ok);
    return ok;
  }

  // ---------------------------------------------- attention compute waves
  // Scores and the weighted sum of values run on the matrix cores with
  // fp32 accumulation.  A wave takes blocks of BP = 16 consecutive cached
  // positions; block t of wave cw starts at position (t*kCW + cw)*BP of its
  // range.  q and the softmax weights p are fp32: each enters the bf16
  // products as three parts (hi, mid, lo), x = hi + mid + lo exactly
  // (split3), one operand row each, and the three rows' results are added,
  // so every product is exact and only the order of the fp32 sums differs
  // from a plain fp32 dot product (the cached k and v are bf16).
  //
  // Scores (v_mfma_f32_16x16x32_bf16, HD/32 steps): D[16 x 16] = K[16 pos x
  // HD] * Qop[HD x 16].  Qop's column 4h + k holds part k of q head h (k = 3:
  // zeros).  Lane l holds D rows 4(l/16)..+3 (positions) of column l%16, so
  // the four lanes of a quad l%16 = 4h..4h+3 hold head h's parts of the same
  // four positions; two DPP steps add them, leaving the score in each.  Those
  // lanes then hold exactly the A operand of the value product
  // (v_mfma_f32_16x16x16_bf16, HD/16 steps): row 4h + k = part k of head
  // h's weights, positions 4(l/16)..+3.  So the weights never leave the
  // registers: O[16 x HD] += P[16 x 16 pos] * V[16 pos x HD], O's rows 4h..4h+2
  // being head h's parts.  The value operand wants four consecutive
  // positions of one dimension per lane, so the V cache is stored in tiles
  // of 4 positions: element (j, e) of a KV head's plane sits at
  // (j/4 * HD + e) * 4 + j%4.
  static constexpr int BP = 16;                // positions per block
  static constexpr int NKC = HD / 32;          // score steps (32 dims each)
  static constexpr int NVC = HD / 16;          // value steps (16 dims each)
  static constexpr int PPB = BP * kCW;         // positions per pass (one block per wave)
  // blocks the home holds in registers, loaded a layer ahead (the split
  // variant's home also gathers and merges the helpers' partials)
  static constexpr int MB = LONG ? 2 : 4;
  static_assert(MB >= 2 && MB % 2 == 0, "the home streams through two of its register blocks; scores go in pairs");
  static_assert(GS == 2 && HD % 32 == 0, "matrix-core attention: two q heads per KV head");

  // x = hi + mid + lo, each a bf16 (bits in the low half), exactly: each
  // part rounds what the previous ones left, and 3 x 8 significant bits
  // cover an fp32 value.
  static __device__ __forceinline__ void split3(float x, uint32_t (&part)[3]) {
    part[0] = f32_to_bf16(x);
    const float r1 = x - bf16_to_f32((uint16_t)part[0]);
    part[1] = f32_to_bf16(r1);
    part[2] = f32_to_bf16(r1 - bf16_to_f32((uint16_t)part[1]));
  }

  struct KVBlock {
    v4u k[NKC];   // A operand of the scores: row j0 + l%16, dims 32c + 8(l/16) .. +7
    v2u v[NVC];   // B operand of the value product: positions j0 + 4(l/16) .. +3 of dim 16c + l%16
  };
  struct KVRegs {
    KVBlock b[MB];
  };

  static __device__ __forceinline__ size_t kv_plane(const Params& p) { return (size_t)((p.max_ctx + 3) & ~3) * HD; }

  // The block at positions j0 .. j0+15 (j0 a multiple of 4).  Rows past
  // `last` read row `last`, and tiles past its tile that tile: finite
  // values, weight 0 at use.
  static __device__ __forceinline__ void kv_block_load(const Params& p, int l, int g, int j0, int last, KVBlock& kb) {
    const int lane = lane_id(), r = lane & 15, q = lane >> 4;
    const size_t plane = kv_plane(p);
    // one buffer resource per plane (base in scalar registers, 32-bit lane offsets)
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.kv + ((size_t)(l * 2 + 0) * p.nkv + g) * plane, (uint32_t)(2 * plane));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.kv + ((size_t)(l * 2 + 1) * p.nkv + g) * plane, (uint32_t)(2 * plane));
    const int lc = max(last, 0);
    const uint32_t ok = 2u * (uint32_t)(min(j0 + r, lc) * HD + 8 * q);
#pragma unroll
    for (int c = 0; c < NKC; ++c)
      kb.k[c] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rk, ok + 64u * c, 0, 0));
    const uint32_t ov = 8u * (uint32_t)(min((j0 >> 2) + q, lc >> 2) * HD + r);
#pragma unroll
    for (int c = 0; c < NVC; ++c)
      kb.v[c] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rv, ov + 128u * c, 0, 0));
  }
  // the home's register blocks cover positions 0 .. MB*PPB-1 of its slice
  static __device__ __forceinline__ void kv_prefetch(const Params& p, int l, int g, int pos, int cw, KVRegs& kv) {
#pragma unroll
    for (int t = 0; t < MB; ++t) kv_block_load(p, l, g, (t * kCW + cw) * BP, pos - 1, kv.b[t]);
  }

  // The q operand (B of the scores) of this lane, from the part rows in LDS.
  static __device__ __forceinline__ void att_qop(const S& s, v4u (&qop)[NKC]) {
    const int lane = lane_id(), r = lane & 15, q = lane >> 4;
    const bool live = r < 4 * GS && (r & 3) != 3;
#pragma unroll
    for (int c = 0; c < NKC; ++c)
      qop[c] = live ? *reinterpret_cast<const v4u*>(&s.qa[r][32 * c + 8 * q]) : v4u{0u, 0u, 0u, 0u};
  }

  // Scores of block j0 in log2 units from its product d: sc[i] for position
  // j0 + 4(l/16) + i of this lane's head ((l%16) / 4), -inf outside [a, b)
  // and in lanes past the two heads' quads.
  static __device__ __forceinline__ void att_score_out(const f4& d, int j0, int a, int b, float (&sc)[4]) {
    const int lane = lane_id(), r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = d[i] + dpp<0xB1>(d[i]);   // (hi + mid), (lo + 0)
      v = v + dpp<0x4E>(v);               // the quad's sum, in every lane of it
      const int j = j0 + 4 * q + i;
      sc[i] = r < 4 * GS && j >= a && j < b ? v : -INFINITY;
    }
  }
  static __device__ __forceinline__ void att_block_scores(const S& s, const KVBlock& kb, int j0, int a, int b,
                                                          float (&sc)[4]) {
    v4u qop[NKC];
    att_qop(s, qop);   // from LDS for every streamed block: no registers held across blocks
    f4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKC; ++c)
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb.k[c]), __builtin_bit_cast(bf16x8, qop[c]),
                                                  d, 0, 0, 0);
    att_score_out(d, j0, a, b, sc);
  }
  // Two held blocks' scores at once (q operand in registers): their
  // matrix-core chains interleave instead of waiting on each other.
  static __device__ __forceinline__ void att_pair_scores(const v4u (&qop)[NKC], const KVBlock& ka, const KVBlock& kb,
                                                         int ja, int jb, int a, int b, float (&sa)[4],
                                                         float (&sb)[4]) {
    f4 da = {0.f, 0.f, 0.f, 0.f}, db = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      da = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka.k[c]), __builtin_bit_cast(bf16x8, qop[c]),
                                                   da, 0, 0, 0);
      db = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb.k[c]), __builtin_bit_cast(bf16x8, qop[c]),
                                                   db, 0, 0, 0);
    }
    att_score_out(da, ja, a, b, sa);
    att_score_out(db, jb, a, b, sb);
  }
  // The entry of a per-head pair (wave-uniform values) for head `odd`.
  // Read out through readfirstlane: a plain select between two array
  // elements is turned into an indexed load from private memory.
  static __device__ __forceinline__ float head_pick(const float (&v)[GS], bool odd) {
    const float v0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v[0])));
    const float v1 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v[1])));
    return odd ? v1 : v0;
  }
  // Maximum of a lane value over head h's lanes (l%16 = 4h), uniform.
  static __device__ __forceinline__ float head_max(float v, int h) {
    return fmaxf(fmaxf(lane_f(v, 4 * h), lane_f(v, 16 + 4 * h)), fmaxf(lane_f(v, 32 + 4 * h), lane_f(v, 48 + 4 * h)));
  }
  static __device__ __forceinline__ float block_max(const float (&sc)[4]) {
    return fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  }
  // Online-softmax step for both heads: fold the candidates bm (uniform)
  // into (m, lsum, acc).  lsum lives in the score lanes (head (l%16)/4), acc
  // rows in the lanes of head l/16.
  static __device__ __forceinline__ void att_rescale(const float (&bm)[GS], float (&m)[GS], float& lsum,
                                                     f4 (&acc)[NVC]) {
    const int lane = lane_id();
    float sc[GS];
#pragma unroll
    for (int h = 0; h < GS; ++h) {
      const float mn = fmaxf(m[h], bm[h]);
      sc[h] = m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - mn);
      m[h] = mn;
    }
    lsum *= head_pick(sc, (lane & 4) != 0);
    const float sa = head_pick(sc, (lane & 16) != 0);
#pragma unroll
    for (int c = 0; c < NVC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[c][i] *= sa;
  }
  // Weights of one block under the maxima m, and the value product.  The
  // lanes of the hi parts add their weights to lsum (each weight once).
  // The parts come from the hardware bf16 pair conversion (round to nearest
  // even), two positions at a time.
  static __device__ __forceinline__ void att_block_accum(const KVBlock& kb, const float (&sc)[4], const float (&m)[GS],
                                                         float& lsum, f4 (&acc)[NVC]) {
    const int k = lane_id() & 3;
    const float mh = head_pick(m, (lane_id() & 4) != 0);
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = sc[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[i] - mh);
      lsum += k == 0 ? pv[i] : 0.f;
    }
    v2u part[3];   // (positions 0,1), (2,3) of each part
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      part[t] = v2u{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
      pv[0] -= bf16_lo(part[t].x);
      pv[1] -= bf16_hi(part[t].x);
      pv[2] -= bf16_lo(part[t].y);
      pv[3] -= bf16_hi(part[t].y);
    }
    // lanes past the two heads' quads have pv = 0: every part is 0
    const v2u pa = k == 0 ? part[0] : (k == 1 ? part[1] : (k == 2 ? part[2] : v2u{0u, 0u}));
#pragma unroll
    for (int c = 0; c < NVC; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, pa), __builtin_bit_cast(s4, kb.v[c]),
                                                         acc[c], 0, 0, 0);
  }
  // One block, streamed: scores, rescale, accumulate.
  static __device__ __forceinline__ void att_block(const S& s, const KVBlock& kb, int j0, int a, int b, float (&m)[GS],
                                                   float& lsum, f4 (&acc)[NVC]) {
    float sc[4];
    att_block_scores(s, kb, j0, a, b, sc);
    const float v = block_max(sc);
    float bm[GS];
#pragma unroll
    for (int h = 0; h < GS; ++h) bm[h] = head_max(v, h);
    att_rescale(bm, m, lsum, acc);
    att_block_accum(kb, sc, m, lsum, acc);
  }
  // Positions [a, b) of the cache, blocks from a0 (a multiple of 4, at most
  // a), one pass of kCW blocks at a time, two blocks in flight in k0 and k1
  // (the home passes two of its register blocks, whose values are used up).
  static __device__ __forceinline__ void att_stream(const Params& p, const S& s, int l, int g, int a0, int a, int b,
                                                    int cw, float (&m)[GS], float& lsum, f4 (&acc)[NVC], KVBlock& k0,
                                                    KVBlock& k1) {
    if (b <= a) return;
    kv_block_load(p, l, g, a0 + cw * BP, b - 1, k0);
    for (int j0 = a0; j0 < b; j0 += 2 * PPB) {
      kv_block_load(p, l, g, j0 + PPB + cw * BP, b - 1, k1);
      att_block(s, k0, j0 + cw * BP, a, b, m, lsum, acc);
      kv_block_load(p, l, g, j0 + 2 * PPB + cw * BP, b - 1, k0);
      att_block(s, k1, j0 + PPB + cw * BP, a, b, m, lsum, acc);
    }
  }
  // att_stream with the first pass's block already issued into k0.
  static __device__ __forceinline__ void att_stream_issued(const Params& p, const S& s, int l, int g, int a0, int a,
                                                           int b, int cw, float (&m)[GS], float& lsum,
                                                           f4 (&acc)[NVC], KVBlock& k0) {
    if (b <= a) return;
    KVBlock k1;
    for (int j0 = a0; j0 < b; j0 += 2 * PPB) {
      kv_block_load(p, l, g, j0 + PPB + cw * BP, b - 1, k1);
      att_block(s, k0, j0 + cw * BP, a, b, m, lsum, acc);
      kv_block_load(p, l, g, j0 + 2 * PPB + cw * BP, b - 1, k0);
      att_block(s, k1, j0 + PPB + cw * BP, a, b, m, lsum, acc);
    }
  }
  // This wave's unnormalised outputs (lanes 16h + i: head h, dims 16c + i),
  // maxima and sums to LDS.
  static __device__ __forceinline__ void att_wave_part(S& s, int cw, const float (&m)[GS], float lsum,
                                                       const f4 (&acc)[NVC]) {
    const int lane = lane_id();
    if (lane < 16 * GS) {
      const int h = lane >> 4, e = lane & 15;
#pragma unroll
      for (int c = 0; c < NVC; ++c) s.part[cw][h * HD + 16 * c + e] = (acc[c][0] + acc[c][1]) + acc[c][2];
    }
#pragma unroll
    for (int h = 0; h < GS; ++h) {
      const float lt =
          (lane_f(lsum, 4 * h) + lane_f(lsum, 16 + 4 * h)) + (lane_f(lsum, 32 + 4 * h) + lane_f(lsum, 48 + 4 * h));
      if (lane == 0) {
        s.wm[cw][h] = m[h];
        s.wl[cw][h] = lt;
      }
    }
  }
  // weight of a partial with maximum mw under the common maximum M
  static __device__ __forceinline__ float att_weight(float mw, float M) {
    return mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
  }

  // Home workgroup of KV head g.  Its slice is positions 0..P-1 of the cache
  // (all of 0..pos-1 without helpers); position `pos` itself (its k and v were
  // produced in this step) enters at the merge, with the helpers' partials.
  static __device__ __forceinline__ bool att_layer(const Params& p, S& s, int l, int g, int pos, int ns, int cw,
                                                   KVRegs& kv, uint32_t epoch, __amdgpu_buffer_rsrc_t rx, bool ok) {
    const int lane = lane_id();
    const int ph = 2 + 6 * l;
    arrive(s, cw, 5u * (uint32_t)l + 1u, false);   // this workgroup stores no q/k/v
    ok = ok && wait_seq(p, &s.seq, (uint32_t)l + 1u);
    XR_MIN(s, ph + 1, XR_SEEN);
    att_prepare<true>(p, s, l, g, pos, cw, ok);
    lds_barrier();
    if (cw == 0) att_current_scores(s);   // read in the merge, after the next barrier
    f4 acc[NVC];
    float m[GS], lsum = 0.f;
#pragma unroll
    for (int h = 0; h < GS; ++h) m[h] = -INFINITY;
#pragma unroll
    for (int c = 0; c < NVC; ++c) acc[c] = f4{0.f, 0.f, 0.f, 0.f};
    const int P = LONG && ns > 0 ? (pos + ns) / (ns + 1) : pos;   // the home's slice: slice 0
    const int nblk = (P + PPB - 1) / PPB;   // passes of one block per wave
    // held blocks of this wave that start before P (its others are all
    // masked: their matrix-core work is skipped, their registers stay
    // loaded).  Only without split attention: there the home's two held
    // blocks are nearly always live, and the branch cost more than it saved.
    const int nblk_w = LONG ? nblk : min(nblk, P > cw * BP ? (P - cw * BP + PPB - 1) / PPB : 0);
#ifdef MK_XRAY
    {  // X-ray: when the prefetched rows are all in registers
      uint32_t z = 0;
#pragma unroll
      for (int t = 0; t < MB; ++t) z ^= kv.b[t].k[0].x ^ kv.b[t].v[NVC - 1].y;
      asm volatile("" ::"v"(z));   // wait until they have arrived
      XR_MAX(s, ph + 1, XR_M0 + 1);
    }
#endif
    // ---- the blocks held in registers (loaded a layer ahead): all scores,
    // one maximum, then the weights and the value products
    if (nblk > 0) {
      v4u qop[NKC];
      att_qop(s, qop);
      float sc[MB][4];
      float v = -INFINITY;
      // in pairs: a block past P scores -inf everywhere (its registers hold
      // finite values), so a pair with one live block still gives the
      // right maximum
#pragma unroll
      for (int t = 0; t < MB; t += 2) {
        if (t < nblk_w) {
          att_pair_scores(qop, kv.b[t], kv.b[t + 1], (t * kCW + cw) * BP, ((t + 1) * kCW + cw) * BP, 0, P, sc[t],
                          sc[t + 1]);
          v = fmaxf(v, fmaxf(block_max(sc[t]), block_max(sc[t + 1])));
        }
      }
      // the first fold: m is -inf and lsum, acc are 0, so the rescale of
      // att_rescale would multiply zeros; take the maxima directly
#pragma unroll
      for (int h = 0; h < GS; ++h) m[h] = head_max(v, h);
#pragma unroll
      for (int t = 0; t < MB; ++t)
        if (t < nblk_w) att_block_accum(kv.b[t], sc[t], m, lsum, acc);
    }
    // ---- longer slices: the remaining blocks stream
    if (nblk > MB) att_stream(p, s, l, g, MB * PPB, MB * PPB, P, cw, m, lsum, acc, kv.b[0], kv.b[1]);
    att_wave_part(s, cw, m, lsum, acc);
    XR_MAX(s, ph + 1, XR_M0);
    lds_barrier();
    // ---- the helpers' partials (split attention): every compute wave
    // gathers a share into LDS; nothing else of this workgroup is in flight
    if (LONG && ns > 0) {
      XR_PUT(s, ph + 2, XR_START);
      const uint32_t pb = xword(p, l, V_ATT) + (uint32_t)(g * p.split_max * p.split_pw);
      const int pw = p.split_pw;
      const __amdgpu_buffer_rsrc_t rs = xch_rsrc(p);
      // rounds of kCW * 64 * KP pairs (registers: one 16-byte load per pair in flight)
      for (int r0 = 0; r0 < ns * PP; r0 += kCW * 64 * KP)
        ok = ok && gather_pairs_to<KP>(
                       p, rs, ns * PP, make_tag(epoch, vec_id(l, V_ATT)),
                       [=](int j) { return pb + (uint32_t)((j / PP) * pw + 2 * (j % PP)); },
                       [&](int j, uint32_t a, uint32_t b) {
                         *reinterpret_cast<v2u*>(&s.spart[j / PP][2 * (j % PP)]) = v2u{a, b};
                       },
                       r0 + cw * 64, kCW * 64);
      XR_MAX(s, ph + 2, XR_READY);
      lds_barrier();
      XR_MIN(s, ph + 2, XR_SEEN);
    }
    // merge the seven waves (fixed order), the helpers and the current
    // position; thread t < NOUT owns output t
    const int t = cw * 64 + lane;
    const int tc = min(t, NOUT - 1);
    const int h = tc / HD;
    // every LDS read of the merge goes out before the first is used
    float wm[kCW], wl[kCW], wp[kCW];
#pragma unroll
    for (int w = 0; w < kCW; ++w) {
      wm[w] = s.wm[w][h];
      wl[w] = s.wl[w][h];
      wp[w] = s.part[w][tc];
    }
    const float sp = s.sp[h];
    const uint32_t vpw = s.vp[(tc % HD) / 2];
    float M = sp;
#pragma unroll
    for (int w = 0; w < kCW; ++w) M = fmaxf(M, wm[w]);
    if (LONG) {
#pragma unroll 8
      for (int i = 0; i < ns; ++i) M = fmaxf(M, s.spart[i][NOUT + h]);
    }
    const float ec = __builtin_amdgcn_exp2f(sp - M);
    float Lt = ec, O = ec * ((tc & 1) ? bf16_hi(vpw) : bf16_lo(vpw));
#pragma unroll
    for (int w = 0; w < kCW; ++w) {
      const float e = att_weight(wm[w], M);
      Lt = fmaf(wl[w], e, Lt);
      O = fmaf(wp[w], e, O);
    }
    if (LONG) {
      // eight partials at a time: their LDS reads all go out before the
      // first is used (rows past the last re-read it and are not added);
      // the sums keep the helpers' order
      for (int i0 = 0; i0 < ns; i0 += 8) {
        float mw[8], lw[8], ow[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = min(i0 + k, ns - 1);
          mw[k] = s.spart[i][NOUT + h];
          lw[k] = s.spart[i][NOUT + GS + h];
          ow[k] = s.spart[i][tc];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (i0 + k < ns) {
            const float e = att_weight(mw[k], M);
            Lt = fmaf(lw[k], e, Lt);
            O = fmaf(ow[k], e, O);
          }
        }
      }
    }
    const float o = O * __builtin_amdgcn_rcpf(Lt);   // v_rcp_f32: within 1 ulp
    XR_MAX(s, ph + 2, XR_M0);
    const float o1 = dpp<0xB1>(o);   // the neighbouring output (t ^ 1)
    st_xword(rx, ok && t < NOUT && (t & 1) == 0 ? 8u * (xword(p, l, V_O) + (g * NOUT + t) / 2) : kOOB,
             pack_bf16(o, o1), make_tag(epoch, vec_id(l, V_O)));
    XR_MAX(s, ph + 1, XR_DONE);
    arrive(s, cw, 5u * (uint32_t)l + 5u, true);   // attention output stored; nothing of the other phases
    lds_barrier();
    // the next layer's held blocks (the last layer reloads its own: one
    // instance of this code for every layer)
    kv_prefetch(p, min(l + 1, p.L - 1), g, pos, cw, kv);
    return ok;
  }

  static __device__ __forceinline__ bool att_waves(const Params& p, S& s, int g, int pos, int ns, int cw,
                                                   uint32_t epoch, __amdgpu_buffer_rsrc_t rx) {
    KVRegs kv;
    kv_prefetch(p, 0, g, pos, cw, kv);
    bool ok = true;
    for (int l = 0; l < p.L; ++l) ok = att_layer(p, s, l, g, pos, ns, cw, kv, epoch, rx, ok);
    return ok;
  }

  // Slice i of KV head g's cached positions for split attention: [a, b).
  static __device__ __forceinline__ void help_slice(int i, int pos, int ns, int& a, int& b) {
    const int chunk = (pos + ns) / (ns + 1);
    a = min(pos, i * chunk);
    b = min(pos, a + chunk);
  }
  // The first pass of a helper's slice, issued before its q is there.
  static __device__ __forceinline__ void help_issue(const Params& p, int l, int g, int i, int pos, int ns, int cw,
                                                    KVBlock& k0) {
    int a, b;
    help_slice(i, pos, ns, a, b);
    if (b <= a) return;
    const int a0 = a & ~3;
    kv_block_load(p, l, g, a0 + cw * BP, b - 1, k0);
  }

  // Split-attention helper (a GEMV workgroup's compute waves, after their
  // QKV rows and before the layer's weight burst): slice i of KV head g's
  // cached positions, merged over the waves and published as (unnormalised
  // outputs, per-head maximum, per-head sum) for the head's home.  k0 holds
  // the slice's first pass (help_issue).
  static __device__ __forceinline__ bool att_help(const Params& p, S& s, int l, int g, int i, int pos, int ns,
                                                  int cw, uint32_t want, uint32_t epoch, __amdgpu_buffer_rsrc_t rx,
                                                  bool ok, KVBlock& k0) {
    const int lane = lane_id();
    const int ph = 2 + 6 * l;
    ok = ok && wait_seq(p, &s.seq, want);
    XR_MIN(s, ph + 1, XR_SEEN);
    att_prepare<false>(p, s, l, g, pos, cw, ok);
    lds_barrier();
    int a, b;
    help_slice(i, pos, ns, a, b);
    f4 acc[NVC];
    float m[GS], lsum = 0.f;
#pragma unroll
    for (int h = 0; h < GS; ++h) m[h] = -INFINITY;
#pragma unroll
    for (int c = 0; c < NVC; ++c) acc[c] = f4{0.f, 0.f, 0.f, 0.f};
    att_stream_issued(p, s, l, g, a & ~3, a, b, cw, m, lsum, acc, k0);
    att_wave_part(s, cw, m, lsum, acc);
    lds_barrier();
    const int t = cw * 64 + lane;
    const int tc = min(t, NOUT - 1);
    const int h = tc / HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kCW; ++w) M = fmaxf(M, s.wm[w][h]);
    float Lt = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kCW; ++w) {
      const float e = att_weight(s.wm[w][h], M);
      Lt = fmaf(s.wl[w][h], e, Lt);
      O = fmaf(s.part[w][tc], e, O);
    }
    const uint32_t base = 8u * (xword(p, l, V_ATT) + (uint32_t)((g * p.split_max + i - 1) * p.split_pw));
    const uint32_t tag = make_tag(epoch, vec_id(l, V_ATT));
    const bool in = ok && t < NOUT;
    st_xword(rx, in ? base + 8u * (uint32_t)t : kOOB, __float_as_uint(O), tag);
    const bool first = in && (t % HD) == 0;   // one thread per head stores its maximum and sum
    st_xword(rx, first ? base + 8u * (uint32_t)(NOUT + h) : kOOB, __float_as_uint(M), tag);
    st_xword(rx, first ? base + 8u * (uint32_t)(NOUT + GS + h) : kOOB, __float_as_uint(Lt), tag);
    XR_MAX(s, ph + 1, XR_DONE);
    return ok;
  }

  // ------------------------------------------------------------ LM head
  // Rows [va, vb) of this workgroup; compute wave cw takes va + cw + 7k, in
  // batches of UBH rows, NBH batches in flight (the first NBH go out before
  // the wait for the final residual).  Returns the wave's best (value,
  // smallest index).  Rows past the wave's last are clamped to it and their
  // results dropped (no branch around a load or a store).
  static constexpr int UBH = F_8 == FMT_BF16 ? 4 : 8;
  // FP8 rows carry a scale register each: two batches in flight (8 rows of
  // 1 KB per wave each, still far more bytes in flight than the HBM latency
  // needs).  With four, the step loop's registers (the GEMV's and the LM
  // head's values live in one loop) no longer fit in 256 VGPRs.
  static constexpr int NBH = F_8 == FMT_BF16 ? 4 : 2;
  static __device__ __forceinline__ bool lm_head(const Params& p, S& s, const int* hdr, int cw, float* d_logits,
                                                 __amdgpu_buffer_rsrc_t rw, bool ok, float& best, int& bidx,
                                                 uint32_t& t_in) {
    const bool l0 = lane_id() == 0;
    const int va = (int)__builtin_amdgcn_readfirstlane(lds_ld(&s.lm_va));
    const int vb = (int)__builtin_amdgcn_readfirstlane(lds_ld(&s.lm_vb));
#ifdef MK_XRAY
    // the record's third mark: this workgroup's rows (va << 32 | count)
    if (cw == 0 && lane_id() == 0) s.xr.v[2 + 6 * p.L][XR_M0 + 2] = (uint64_t)va << 32 | (uint32_t)(vb - va);
#endif
    const int n = vb > va + cw ? (vb - va - cw + kCW - 1) / kCW : 0;   // rows of this wave
    const GMat g = gmat(p.embed, 0);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(d_logits, d_logits ? 4u * (uint32_t)p.V : 0u);
    auto row = [&](int k) { return n > 0 ? va + cw + kCW * min(k, n - 1) : -1; };
    WRow<F_8, NH> B[NBH][UBH];
#pragma unroll
    for (int q = 0; q < NBH; ++q)
#pragma unroll
      for (int b = 0; b < UBH; ++b) wrow_load(rw, g, row(q * UBH + b), B[q][b]);
    asm volatile("" ::: "memory");
    ok = ok && wait_seq(p, &s.seq, (uint32_t)(p.L * (LONG ? hdr[S_NIN_L] : hdr[S_NIN])) + 1u);
    t_in = (uint32_t)__builtin_amdgcn_s_memrealtime();
    XR_MIN(s, 2 + 6 * p.L, XR_SEEN);
    uint32_t xa[NH][8];
    load_act<NH>(s.xd_act, p.H, xa);
    best = -INFINITY;
    bidx = 0x7FFFFFFF;
    auto use = [&](const WRow<F_8, NH>(&Bq)[UBH], int k0) {
#pragma unroll
      for (int b = 0; b < UBH; ++b) {
        const float v = wrow_dot(Bq[b], xa);
        const bool in = k0 + b < n;
        const int r = va + cw + kCW * (k0 + b);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rl, in && l0 ? 4u * (uint32_t)r : kOOB, 0, 0);
        const bool take = in && v > best;   // a wave's rows ascend, so the first maximum is kept
        best = take ? v : best;
        bidx = take ? r : bidx;
      }
    };
    // each batch is reloaded right after its use; the scheduling barriers
    // keep the loads ahead of the next batch's arithmetic
    for (int k0 = 0; k0 < n; k0 += NBH * UBH) {
#pragma unroll
      for (int q = 0; q < NBH; ++q) {
        use(B[q], k0 + q * UBH);
#pragma unroll
        for (int b = 0; b < UBH; ++b) wrow_load(rw, g, row(k0 + (q + NBH) * UBH + b), B[q][b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    XR_MAX(s, 2 + 6 * p.L, XR_DONE);
    return ok;
  }

  // -------------------------------------------------------------- kernel
  // `nsteps` greedy steps at positions pos0, pos0 + 1, ...: step i runs with
  // exchange epoch epoch0 + i, and its argmax, reduced by every workgroup,
  // is step i + 1's token (d_next[i] gets it too; d_logits, if given, row i
  // the logits).  Between steps the workgroup's waves meet at a barrier,
  // and a failed step stops every wave there.  With nsteps > 1, ns must be
  // 0: a KV row written in one step is read in the next only by the
  // workgroup that wrote it (same CU), while a split-attention helper on
  // another CU could read a stale copy of it (the kernel boundary is what
  // makes earlier launches' rows visible to every CU).
  // One step's state, from LDS.
  struct Step {
    int i, pos;
    uint32_t epoch;
  };
  static __device__ __forceinline__ Step step_state(const S& s) {
    Step t;
    t.i = (int)__builtin_amdgcn_readfirstlane(lds_ld(&s.st_i));
    t.pos = (int)__builtin_amdgcn_readfirstlane(lds_ld(&s.st_pos0)) + t.i;
    t.epoch = __builtin_amdgcn_readfirstlane(lds_ld(&s.st_e0)) + (uint32_t)t.i;
    return t;
  }
  template <typename T>
  static __device__ __forceinline__ T* lds_ptr(const uint32_t (&w)[2]) {
    // each half widened as unsigned (readfirstlane returns a signed int)
    const uint64_t a = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(lds_ld(&w[1])) << 32 |
                       (uint32_t)__builtin_amdgcn_readfirstlane(lds_ld(&w[0]));
    return reinterpret_cast<T*>((uintptr_t)a);
  }
  // Entries [off, off + N) of the workgroup's table row, read anew by every
  // step: nothing derived from them is computed once before the step loop
  // and held (or spilled) across the whole step.
  template <int N>
  static __device__ __forceinline__ void tab_row(const S& s, int off, int (&a)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) a[i] = (int)__builtin_amdgcn_readfirstlane(lds_ld((const uint32_t*)&s.tab[off + i]));
  }
  static __device__ __forceinline__ bool last_step(const S& s, int i) {
    return i + 1 >= (int)__builtin_amdgcn_readfirstlane(lds_ld(&s.st_n));
  }
  // The end of a step with another to follow: a failure in any wave stops
  // every wave; else thread 0 moves the step state on and the counters and
  // records are cleared once every wave is past the step.  Returns true to
  // go on.
  static __device__ __forceinline__ bool step_end(S& s, bool ok) {
    if (!ok && lane_id() == 0) lds_st(&s.fail, 1u);
    lds_barrier();
    if (__builtin_amdgcn_readfirstlane(lds_ld(&s.fail)) != 0) return false;
    if (threadIdx.x == 0) {
      s.seq = 0;
      lds_st(&s.st_i, lds_ld(&s.st_i) + 1u);
#pragma unroll
      for (int w = 0; w < kCW; ++w) lds_st(&s.arr[w], 0u);   // constant offsets, one word each: nothing held across the step
    }
    XR_INIT(s);
    lds_barrier();
    return true;
  }

  // The compute waves' steps: `layers(t, hdr, rx, rw)` runs a step's layers
  // (attention or GEMV units, by the workgroup's role), then the LM head
  // and the workgroup's argmax candidate; `next(rw)` runs when another step
  // follows, before the waves wait for its token.  Each role has its own
  // loop, so the values either role derives once (lane masks, offsets) are
  // held only where that role runs.
  template <typename F, typename G>
  static __device__ __forceinline__ void compute_steps(const Params& p, S& s, int cw, F&& layers, G&& next) {
    const int lane = lane_id(), wg = blockIdx.x;
    for (;;) {
      const Step t = step_state(s);
      int hdr[kHdrInts];
      tab_row(s, 0, hdr);
      const __amdgpu_buffer_rsrc_t rx = xch_rsrc(p);
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w, p.w_bytes);
      bool ok = layers(t, hdr, rx, rw);
      float best;
      int bidx;
      float* lg = lds_ptr<float>(s.st_logits);
      uint32_t t_in;
      ok = lm_head(p, s, hdr, cw, lg ? lg + (size_t)t.i * p.V : nullptr, rw, ok, best, bidx, t_in);
      if (lane == 0) {
        s.best[cw] = best;
        s.bidx[cw] = bidx;
      }
      lds_barrier();
      if (cw == 0) {
        // workgroup argmax: largest value, then smallest index
        float b = s.best[0];
        int bi = s.bidx[0];
#pragma unroll
        for (int w = 1; w < kCW; ++w)
          if (s.best[w] > b || (s.best[w] == b && s.bidx[w] < bi)) {
            b = s.best[w];
            bi = s.bidx[w];
          }
        // the workgroup's record: its (value, index), then when its LM head
        // ended, how long it took (ticks from its input to its last
        // candidate), for how many rows, on which XCD: every workgroup derives
        // the next step's LM-head rows from them
        const uint32_t t_end = (uint32_t)__builtin_amdgcn_s_memrealtime();
        const uint32_t dt = min(t_end - t_in, 0xFFFFu);
        const uint32_t rows = min(lds_ld(&s.lm_vb) - lds_ld(&s.lm_va), 0xFFFu);
        const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7u;   // XCC_ID
        const uint32_t tag = make_tag(t.epoch, vec_id(p.L, 0));
        const uint32_t off = 8u * (uint32_t)(p.x.arg + 4ull * wg);
        st_xword(rx, ok && lane == 0 ? off : kOOB, __float_as_uint(b), tag);
        st_xword(rx, ok && lane == 0 ? off + 8u : kOOB, (uint32_t)bi, tag);
        st_xword(rx, ok && lane == 0 ? off + 16u : kOOB, t_end, tag);
        st_xword(rx, ok && lane == 0 ? off + 24u : kOOB, dt << 16 | rows << 4 | xcc, tag);
      }
      arrive(s, cw, 5u * (uint32_t)p.L + 1u, cw == 0);
      if (last_step(s, t.i)) break;
      next(rw);
      if (!step_end(s, ok)) break;
    }
  }

  static __device__ __forceinline__ void run(const Params& p, S& s, const int32_t* d_token, int pos0, int nsteps,
                                             int ns, uint32_t epoch0, int32_t* d_next, float* d_logits) {
    const int wave = wave_id(), lane = lane_id();
    const int wg = blockIdx.x;
    const int token = __builtin_amdgcn_readfirstlane(*d_token);
    if (token < 0 || token >= p.V) {
      if (wg == 0 && threadIdx.x == 0) {
        raise_error(p, ERR_TOKEN);
        for (int i = 0; i < nsteps; ++i) d_next[i] = -1;
      }
      return;
    }
    if (wg == 0 && threadIdx.x == 0)
      for (int i = 0; i < nsteps; ++i) d_next[i] = -1;   // overwritten on success
    if (threadIdx.x == 0) {
      s.seq = 0;
      s.fail = 0;
      s.st_i = 0;
      s.st_n = (uint32_t)nsteps;
      s.st_pos0 = (uint32_t)pos0;
      s.st_e0 = epoch0;
      s.st_token = (uint32_t)token;
      s.st_next[0] = (uint32_t)(uintptr_t)d_next;
      s.st_next[1] = (uint32_t)((uint64_t)(uintptr_t)d_next >> 32);
      s.st_logits[0] = (uint32_t)(uintptr_t)d_logits;
      s.st_logits[1] = (uint32_t)((uint64_t)(uintptr_t)d_logits >> 32);
      // the first step's LM-head rows: an equal share
      s.lm_va = (uint32_t)((int64_t)p.V * wg / p.grid);
      s.lm_vb = (uint32_t)((int64_t)p.V * (wg + 1) / p.grid);
    }
    if (threadIdx.x < kCW) s.arr[threadIdx.x] = 0;
    XR_INIT(s);
    // this workgroup's row of the work table
    MK_GLOBAL const int* tab = GCAST(const int, p.w + p.sched) + (size_t)wg * kSchedInts * kWaves;
    for (int i = threadIdx.x; i < kWaves * kSchedInts; i += kThreads) s.tab[i] = tab[i];
    lds_barrier();   // seq, the step state, the table row and the X-ray records are initialised
    if (wave == 0) {
      for (;;) {
        const Step t = step_state(s);
        int hdr[kHdrInts];
        tab_row(s, 0, hdr);
        const bool more = !last_step(s, t.i);
        int next = -1;
        bool ok = courier(p, s, hdr, (int)__builtin_amdgcn_readfirstlane(lds_ld(&s.st_token)), t.pos, ns, t.epoch,
                          lds_ptr<int32_t>(s.st_next) + t.i, more, t.i > 0, next);
        // the next step's token is this step's argmax: checked as a launch
        // checks the token it reads (an index past the vocabulary would
        // address past the embedding table)
        if (ok && more && (next < 0 || next >= p.V)) {
          if (lane == 0) raise_error(p, ERR_TOKEN);
          ok = false;
        }
        // A courier that gave up inside the step has handed the abort value
        // to the compute waves (their waits return at once, and they stop at
        // the step's end) and may have skipped barriers of the step: it ends
        // here.  A failed final argmax skipped none: it meets the compute
        // waves at the step's end like a good step.
        if (!ok && __builtin_amdgcn_readfirstlane(lds_ld(&s.seq)) == kAbort) return;
        if (lane == 0) lds_st(&s.st_token, (uint32_t)next);
        if (!more || !step_end(s, ok)) break;
      }
    } else if (s.tab[S_ATT] >= 0) {
      const int g = s.tab[S_ATT];
      compute_steps(
          p, s, wave - 1,
          [&](const Step& t, const int*, __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t) {
            return att_waves(p, s, g, t.pos, ns, wave - 1, t.epoch, rx);
          },
          [](__amdgpu_buffer_rsrc_t) {});
    } else {
      // bf16: layer 0's QKV rows, the first step's now, every later step's
      // while the step before it reduces its argmax (the rows are the same
      // in every step)
      GemvW w;
      auto qkv0 = [&](__amdgpu_buffer_rsrc_t rw) {
        if constexpr (kQKV0Early) {
          int u[kUnitInts];
          tab_row(s, kSchedInts * wave, u);
          load_layer_qkv(p, rw, u, 0, w);
        }
      };
      qkv0(make_rsrc(p.w, p.w_bytes));
      compute_steps(
          p, s, wave - 1,
          [&](const Step& t, const int* hdr, __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw) {
            int u[kUnitInts];
            tab_row(s, kSchedInts * wave, u);
            return gemv_waves(p, s, hdr, u, t.pos, ns, wave - 1, t.epoch, rw, rx, w);
          },
          qkv0);
    }
#ifdef MK_XRAY
    __syncthreads();
    XR_DUMP(s, p);
#endif
  }
};

// One instantiation per (weight format, head_dim, q heads per KV head,
// 1024-chunks of hidden, of n_q_heads*head_dim and of intermediate, split
// attention or not): the formats, the attention shape and every per-lane
// register array size are compile-time constants.  `ns` is the number of
// helpers per KV head in this step (0 without split attention).
template <int WF, int HD, int GS, int NH, int NQ, int NI, bool LONG, bool BAR>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(const Params* __restrict__ pp, const int32_t* d_token,
                                                             int pos, int nsteps, int ns, uint32_t epoch,
                                                             int32_t* d_next, float* d_logits) {
  __shared__ Smem<HD, GS, NH, NQ, NI> s;
  Kern<WF, HD, GS, NH, NQ, NI, LONG, BAR>::run(*pp, s, d_token, pos, nsteps, ns, epoch, d_next, d_logits);
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

// variant: 0 the headline kernel, 1 split attention, 2 grid barriers
static const void* decode_fn(int wfmt, int hd, int gs, int hidden, int qdim, int inter, int variant) {
  const void* fn = nullptr;
  const int nh = cdiv1024(hidden), nqd = cdiv1024(qdim), ni = cdiv1024(inter);
#define MK_FN(W_, H_, G_, A_, B_, C_)                                                                  \
  (variant == 1   ? reinterpret_cast<const void*>(decode_kernel<W_, H_, G_, A_, B_, C_, true, false>)   \
   : variant == 2 ? reinterpret_cast<const void*>(decode_kernel<W_, H_, G_, A_, B_, C_, false, true>)   \
                  : reinterpret_cast<const void*>(decode_kernel<W_, H_, G_, A_, B_, C_, false, false>))
#define MK_CASE(H_, G_, A_, B_, C_)                                                                 \
  if (hd == H_ && gs == G_ && nh == A_ && nqd == B_ && ni == C_) {                                  \
    fn = wfmt == 0 ? MK_FN(0, H_, G_, A_, B_, C_) : (wfmt == 1 ? MK_FN(1, H_, G_, A_, B_, C_)       \
                                                               : MK_FN(2, H_, G_, A_, B_, C_));     \
  }
  MK_SHAPES(MK_CASE)
#undef MK_CASE
#undef MK_FN
  return fn;
}

hipError_t decode_coresident(int wfmt, int hd, int gs, int hidden, int qdim, int inter, int* per_cu) {
  int n[3];
  for (int v = 0; v < 3; ++v) {
    const void* fn = decode_fn(wfmt, hd, gs, hidden, qdim, inter, v);
    if (!fn) return hipErrorInvalidValue;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n[v], fn, kThreads, 0);
    if (e != hipSuccess) return e;
  }
  *per_cu = std::min(n[0], std::min(n[1], n[2]));
  return hipSuccess;
}

hipError_t launch_decode(const Params* d_params, int wfmt, int hd, int gs, int hidden, int qdim, int inter, int grid,
                         bool cooperative, bool barrier, const int32_t* d_token, int pos, int nsteps, int ns,
                         uint32_t epoch, int32_t* d_next, float* d_logits, hipStream_t s) {
  if (barrier && ns > 0) return hipErrorInvalidValue;
  const void* fn = decode_fn(wfmt, hd, gs, hidden, qdim, inter, barrier ? 2 : (ns > 0 ? 1 : 0));
  if (!fn) return hipErrorInvalidValue;
  if (nsteps < 1) return hipErrorInvalidValue;
  void* args[] = {&d_params, &d_token, &pos, &nsteps, &ns, &epoch, &d_next, &d_logits};
  if (cooperative) return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

}  // namespace mk
