// Batched prefill for gfx950: a prompt's positions run through each layer
// together, in chunks of up to kPrefillChunk positions, so the projections are
// matrix-matrix products on the matrix cores (bf16 operands, fp32
// accumulation) instead of one decode launch per position.  Every step keeps
// the decode path's rounding points (GEMM inputs, K, V and the attention
// output in bf16; residuals, q and logits in fp32) and writes the same KV
// cache, so a decode step may follow at position n.
//
// Per chunk of positions [c0, c0 + cn):
//   embed -> per layer: RMSNorm -> QKV GEMM -> q/k RMSNorm, RoPE, KV append ->
//   causal attention over the cache (matrix cores) -> O GEMM + residual -> RMSNorm ->
//   gate/up GEMM + SwiGLU -> down GEMM + residual
// then, after the last chunk, the final RMSNorm, the LM head of the last
// position and its argmax.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <stdint.h>

#include "mk_codec.h"
#include "mk_launch.h"
#include "mk_shared.h"

namespace mk {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef short s4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane() { return (int)(threadIdx.x & 63); }
__device__ __forceinline__ int wave() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t arena(const Params& p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>((const uint8_t*)p.w), (short)0, (int)p.w_bytes,
                                           0x00020000);
}
__device__ __forceinline__ float gain(__amdgpu_buffer_rsrc_t rw, uint64_t off, int i) {
  return bf16_to_f32((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rw, (uint32_t)(off + 2ull * i), 0, 0));
}
__device__ __forceinline__ size_t kv_plane(const Params& p, int hd) { return (size_t)((p.max_ctx + 3) & ~3) * hd; }

// ------------------------------------------------------------------ embed
// X[i, :] = the token's embedding row (bf16, or FP8 codes times the row scale).
__global__ __launch_bounds__(256) void pf_embed(const Params* pp, const int32_t* tokens, int cn, float* X) {
  const Params& p = *pp;
  const int i = blockIdx.x;
  if (i >= cn) return;
  const __amdgpu_buffer_rsrc_t rw = arena(p);
  const uint32_t t = (uint32_t)tokens[i];
  const int H = p.H;
  if (p.embed.fmt == FMT_BF16) {
    for (int e = threadIdx.x; e < H; e += blockDim.x)
      X[(size_t)i * H + e] = gain(rw, p.embed.codes + 2ull * t * H, e);
  } else {
    const float sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, (uint32_t)(p.embed.scales + 4ull * t), 0, 0));
    for (int e = threadIdx.x; e < H; e += blockDim.x) {
      const uint32_t c = __builtin_amdgcn_raw_buffer_load_b8(rw, (uint32_t)(p.embed.codes + (uint64_t)t * H + e), 0, 0);
      X[(size_t)i * H + e] = e4m3_to_f32(c) * sc;
    }
  }
}

// ---------------------------------------------------------------- RMSNorm
// A[i, :] = bf16(g * (x * r)), r = 1/sqrt(mean(x^2) + eps); one workgroup per row.
__global__ __launch_bounds__(256) void pf_rmsnorm(const Params* pp, const float* X, int cn, int H, uint64_t g_off,
                                                  uint16_t* A) {
  const Params& p = *pp;
  __shared__ float red[4];
  const int i = blockIdx.x;
  if (i >= cn) return;
  const float* x = X + (size_t)i * H;
  float ss = 0.f;
  for (int e = threadIdx.x; e < H; e += blockDim.x) ss += x[e] * x[e];
  ss = wsum(ss);
  if (lane() == 0) red[wave()] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float r = 1.0f / sqrtf(tot / (float)H + p.eps);
  const __amdgpu_buffer_rsrc_t rw = arena(p);
  for (int e = threadIdx.x; e < H; e += blockDim.x) {
    const float v = gain(rw, g_off, e) * (x[e] * r);
    A[(size_t)i * H + e] = (uint16_t)f32_to_bf16(v);
  }
}

// ------------------------------------------------------------------- GEMM
// C[M x N] = A[M x K] (bf16, row-major) * W[N x K]^T, W dequantized to bf16
// exactly in registers (FP8 codes; FP4 codes times their E4M3 block scale),
// then each column n times its row scale (FP8) or tensor scale (FP4).  A
// 256-thread workgroup computes a 64 x 64 tile; wave w the 32 x 32 quarter
// (w&1, w>>1) as 2 x 2 v_mfma_f32_16x16x32_bf16 tiles; K in steps of 32
// through LDS.  Epilogues: store C (fp32), add C into the residual X, or
// SwiGLU over interleaved (gate, up) column pairs into bf16 H.
enum : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_PARTIAL = 3 };
constexpr int BK = 32, LDA = BK + 8;

template <uint32_t FMT>
__device__ __forceinline__ u4 load_w8(__amdgpu_buffer_rsrc_t rw, const Mat& m, uint64_t lo, int n, int k) {
  // 8 consecutive weights (n, k..k+7) as bf16; n < N and k + 8 <= K (callers clamp)
  const uint64_t el = (uint64_t)n * m.K + k;
  if (FMT == FMT_BF16) {
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rw, (uint32_t)(m.codes + lo + 2 * el), 0, 0));
  } else if (FMT == FMT_FP8) {
    const u2 c = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rw, (uint32_t)(m.codes + lo + el), 0, 0));
    return u4{e4m3x2_to_bf16x2<false>(c.x), e4m3x2_to_bf16x2<true>(c.x), e4m3x2_to_bf16x2<false>(c.y),
              e4m3x2_to_bf16x2<true>(c.y)};
  } else {
    const uint32_t c = __builtin_amdgcn_raw_buffer_load_b32(rw, (uint32_t)(m.codes + lo + el / 2), 0, 0);
    const uint32_t bs = __builtin_amdgcn_raw_buffer_load_b8(rw, (uint32_t)(m.scales + lo + el / 16), 0, 0);
    const float s = e4m3_to_f32(bs);
    const uint32_t w2[4] = {e2m1x2_to_bf16x2<0>(c), e2m1x2_to_bf16x2<1>(c), e2m1x2_to_bf16x2<2>(c),
                            e2m1x2_to_bf16x2<3>(c)};
    u4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // e2m1 * e4m3 has at most 6 significant bits: exact in bf16
      const uint32_t v = pack_bf16(bf16_lo(w2[j]) * s, bf16_hi(w2[j]) * s);
      o[j] = v;
    }
    return o;
  }
}

template <uint32_t FMT>
__device__ __forceinline__ float col_scale(__amdgpu_buffer_rsrc_t rw, const Mat& m, uint64_t lo, int n) {
  if (FMT == FMT_FP8)
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, (uint32_t)(m.scales + lo + 4ull * n), 0, 0));
  if (FMT == FMT_FP4) {
    uint32_t idx = 0;
    if (m.ts_mode == 1) idx = (uint32_t)n < m.ts_b0 ? 0u : ((uint32_t)n < m.ts_b1 ? 1u : 2u);
    else if (m.ts_mode == 2) idx = (uint32_t)n & 1u;
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, (uint32_t)(m.tscale + lo + 4ull * idx), 0, 0));
  }
  return 1.0f;
}

template <uint32_t FMT, int EPI, int T>
__global__ __launch_bounds__(256) void pf_gemm(const Params* pp, const Mat* mat, uint64_t lo, const uint16_t* A, int M,
                                               float* C, uint16_t* Hout) {
  // T x T tile: each wave owns a (T/2) x (T/2) quarter of (T/32)^2 MFMA
  // tiles.  K advances by KS = 2 * BK per stage: two LDS buffers (one
  // barrier per stage) fed from three stages of operands in registers, so
  // global loads are issued three stages ahead of their use.
  constexpr int NT = T / 32, KS = 2 * BK, LDK = KS + 8;
  constexpr int RP = T >= 64 ? T / 64 : 1;   // rows a thread stages
  constexpr int OPB = 2 * 2 * T * LDK * 2, EPB = T * (T + 1) * 4;
  const Params& p = *pp;
  const Mat m = *mat;
  const int N = (int)m.N, K = (int)m.K;
  // the operand buffers (two stages of A and W) and, after the main loop,
  // the fp32 tile for the epilogue share one LDS block
  __shared__ __attribute__((aligned(16))) uint8_t smem[OPB > EPB ? OPB : EPB];
  uint16_t(*sa)[T][LDK] = reinterpret_cast<uint16_t(*)[T][LDK]>(smem);
  uint16_t(*sw)[T][LDK] = sa + 2;
  float(*sc)[T + 1] = reinterpret_cast<float(*)[T + 1]>(smem);
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  const int t = threadIdx.x, w = wave(), l = lane();
  const __amdgpu_buffer_rsrc_t rw = arena(p);
  // thread t < 4T stages rows t/4 + 64i, columns 8*(t%4) and 32 + 8*(t%4) of a stage
  const bool stager = t < 4 * T;
  const int sk = 8 * (t & 3);
  int srw[RP], am[RP], wn[RP];
#pragma unroll
  for (int i = 0; i < RP; ++i) {
    srw[i] = min((t >> 2) + 64 * i, T - 1);
    am[i] = min(m0 + srw[i], M - 1);
    wn[i] = min(n0 + srw[i], N - 1);
  }
  f4v acc[NT][NT];
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f4v{0.f, 0.f, 0.f, 0.f};
  const int wr = (T / 2) * (w & 1), wc = (T / 2) * (w >> 1);
  // split K (EPI_PARTIAL): workgroup z sums K range [z*K/Z, (z+1)*K/Z); the
  // range is a multiple of KS (host)
  const int kz = K / (int)gridDim.z, kbeg = (int)blockIdx.z * kz, nst = kz / KS;
  // stage operands in registers, three stages in flight (a ring of three,
  // the loop unrolled by three so every index is static)
  struct Stage {
    u4 a0[RP], a1[RP], w0[RP], w1[RP];
  };
  auto load = [&](int stg, Stage& r) {
    const int k = kbeg + stg * KS;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const uint16_t* arow = A + (size_t)am[i] * K;
      r.a0[i] = *reinterpret_cast<const u4*>(arow + k + sk);
      r.a1[i] = *reinterpret_cast<const u4*>(arow + k + BK + sk);
      r.w0[i] = load_w8<FMT>(rw, m, lo, wn[i], k + sk);
      r.w1[i] = load_w8<FMT>(rw, m, lo, wn[i], k + BK + sk);
    }
  };
  auto put = [&](const Stage& r, int buf) {
    if (stager) {
#pragma unroll
      for (int i = 0; i < RP; ++i) {
        *reinterpret_cast<u4*>(&sa[buf][srw[i]][sk]) = r.a0[i];
        *reinterpret_cast<u4*>(&sa[buf][srw[i]][BK + sk]) = r.a1[i];
        *reinterpret_cast<u4*>(&sw[buf][srw[i]][sk]) = r.w0[i];
        *reinterpret_cast<u4*>(&sw[buf][srw[i]][BK + sk]) = r.w1[i];
      }
    }
  };
  auto mul = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < KS; kk += BK) {
#pragma unroll
      for (int a = 0; a < NT; ++a) {
        const u4 ao = *reinterpret_cast<const u4*>(&sa[buf][wr + 16 * a + (l & 15)][kk + 8 * (l >> 4)]);
#pragma unroll
        for (int b = 0; b < NT; ++b) {
          const u4 bo = *reinterpret_cast<const u4*>(&sw[buf][wc + 16 * b + (l & 15)][kk + 8 * (l >> 4)]);
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, ao), __builtin_bit_cast(bf8v, bo),
                                                              acc[a][b], 0, 0, 0);
        }
      }
    }
  };
  // step s: multiply stage s (LDS buffer s&1), move stage s+1 (registers,
  // ring slot (s+1)%3) to the other buffer, load stage s+3 into slot s%3
  auto step = [&](int st, Stage& nxt, Stage& freed) {
    if (st < nst) {   // uniform
      mul(st & 1);
      if (st + 1 < nst) put(nxt, (st + 1) & 1);
      if (st + 3 < nst) load(st + 3, freed);
      __syncthreads();
    }
  };
  Stage r0, r1, r2;
  load(0, r0);
  if (nst > 1) load(1, r1);
  if (nst > 2) load(2, r2);
  put(r0, 0);
  __syncthreads();
  for (int st = 0; st < nst; st += 3) {
    step(st, r1, r0);
    step(st + 1, r2, r1);
    step(st + 2, r0, r2);
  }
  // D: lane l holds rows 4(l/16)+i of column l%16 of each 16 x 16 tile
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int cc = wc + 16 * b + (l & 15);
      const float s = col_scale<FMT>(rw, m, lo, min(n0 + cc, N - 1));
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[wr + 16 * a + 4 * (l >> 4) + i][cc] = acc[a][b][i] * s;
    }
  __syncthreads();
  if (EPI == EPI_SWIGLU) {
    // columns (2j, 2j+1) = (gate j, up j): h_j = silu(gate) * up, bf16
    const int I = N / 2;
    for (int e = t; e < T * T / 2; e += 256) {
      const int r = e / (T / 2), j = e % (T / 2);
      const int gm = m0 + r, gj = n0 / 2 + j;
      if (gm < M && gj < I) Hout[(size_t)gm * I + gj] = (uint16_t)f32_to_bf16(silu_f(sc[r][2 * j]) * sc[r][2 * j + 1]);
    }
  } else {
    for (int e = t; e < T * T; e += 256) {
      const int r = e / T, c = e % T;
      const int gm = m0 + r, gn = n0 + c;
      if (gm < M && gn < N) {
        if (EPI == EPI_STORE) C[(size_t)gm * N + gn] = sc[r][c];
        else if (EPI == EPI_PARTIAL) C[((size_t)blockIdx.z * M + gm) * N + gn] = sc[r][c];
        else C[(size_t)gm * N + gn] += sc[r][c];
      }
    }
  }
}

// -------------------------------------------- q/k RMSNorm, RoPE, KV append
// One wave per (position, head slot): slots 0..nq-1 q heads (normed, roped,
// times log2(e)/sqrt(hd), written back in place), nq..nq+nkv-1 k heads
// (normed, roped, bf16, appended), then the v heads (bf16, appended).  Lane
// i < hd/2 owns the RoPE pair (i, i + hd/2).
__global__ __launch_bounds__(256) void pf_qkv_post(const Params* pp, int l, int c0, int cn, float* QKV) {
  const Params& p = *pp;
  const int hd = p.hd, nq = p.nq, nkv = p.nkv, slots = nq + 2 * nkv;
  const int idx = blockIdx.x * 4 + wave();
  if (idx >= cn * slots) return;
  const int i = idx / slots, h = idx % slots, pos = c0 + i;
  const int ln = lane(), li = min(ln, hd / 2 - 1);
  const bool pl = ln < hd / 2;
  float* x = QKV + (size_t)i * slots * hd + (size_t)h * hd;
  const float xa = pl ? x[li] : 0.f, xb = pl ? x[li + hd / 2] : 0.f;
  const size_t plane = kv_plane(p, hd);
  if (h >= nq + nkv) {   // v: round and append (V planes are tiled by 4 positions)
    const int g = h - nq - nkv;
    uint16_t* vc = p.kv + ((size_t)(l * 2 + 1) * nkv + g) * plane;
    if (pl) {
      vc[((size_t)(pos >> 2) * hd + li) * 4 + (pos & 3)] = (uint16_t)f32_to_bf16(xa);
      vc[((size_t)(pos >> 2) * hd + li + hd / 2) * 4 + (pos & 3)] = (uint16_t)f32_to_bf16(xb);
    }
    return;
  }
  const __amdgpu_buffer_rsrc_t rw = arena(p);
  const uint64_t lo = (uint64_t)l * p.layer_stride;
  const bool isq = h < nq;
  const uint64_t goff = (isq ? p.layer0.q_norm : p.layer0.k_norm) + lo;
  const float r = 1.0f / sqrtf(wsum(xa * xa + xb * xb) / (float)hd + p.eps);
  const float a = gain(rw, goff, li) * (xa * r), b = gain(rw, goff, li + hd / 2) * (xb * r);
  const float cs = p.rope[((size_t)pos * (hd / 2) + li) * 2], sn = p.rope[((size_t)pos * (hd / 2) + li) * 2 + 1];
  const float ra = a * cs - b * sn, rb = b * cs + a * sn;
  if (isq) {
    const float kq = 1.4426950408889634f / sqrtf((float)hd);
    if (pl) {
      x[li] = ra * kq;
      x[li + hd / 2] = rb * kq;
    }
  } else {
    const int g = h - nq;
    uint16_t* kc = p.kv + ((size_t)(l * 2 + 0) * nkv + g) * plane + (size_t)pos * hd;
    if (pl) {
      kc[li] = (uint16_t)f32_to_bf16(ra);
      kc[li + hd / 2] = (uint16_t)f32_to_bf16(rb);
    }
  }
}

// --------------------------------------------- attention on the matrix cores
// x = hi + mid + lo exactly, each a bf16 (bits in the low half): each part
// rounds what the previous ones left; 3 x 8 significant bits cover fp32.
__device__ __forceinline__ void split3(float x, uint32_t (&part)[3]) {
  part[0] = f32_to_bf16(x);
  const float r1 = x - bf16_to_f32((uint16_t)part[0]);
  part[1] = f32_to_bf16(r1);
  part[2] = f32_to_bf16(r1 - bf16_to_f32((uint16_t)part[1]));
}

// One workgroup per (block of 16 chunk positions, q head); its 4 waves take
// every 4th block of 16 cached keys and merge their partial softmax states
// in LDS (fixed order).  Per key block, transposed so that the weights stay
// in registers:
//   S^T[16 keys x 16 queries] = K[16 x HD] * Q^T (v_mfma_f32_16x16x32_bf16;
//     q enters as its three exact bf16 parts, three products per step);
//   lane l then holds query l%16's scores for keys 4(l/16)..+3: exactly the
//   B operand of O^T[HD x 16 queries] += V^T[HD x 16 keys] * P^T
//     (v_mfma_f32_16x16x16_bf16, the weights in three exact parts), whose A
//     operand is four consecutive keys of one dimension: one 4-position V tile.
template <int HD>
__global__ __launch_bounds__(256) void pf_attention_mc(const Params* pp, int l, int c0, int cn, const float* QKV,
                                                       uint16_t* O) {
  constexpr int NKC = HD / 32, NVC = HD / 16;
  const Params& p = *pp;
  const int nq = p.nq, nkv = p.nkv, slots = nq + 2 * nkv;
  __shared__ float sm[4][16], sl[4][16];
  __shared__ float so[4][16][HD + 1];
  const int w = wave(), ln = lane(), r = ln & 15, qg = ln >> 4;
  // the last query blocks see the most keys: they go out first, so that the
  // short ones fill in behind them
  const int qb = (int)(gridDim.x / nq) - 1 - (int)(blockIdx.x / nq), h = blockIdx.x % nq, g = h / (nq / nkv);
  const int i0 = 16 * qb;
  const int qi = i0 + r;                       // this lane's query (column)
  const bool qv = qi < cn;
  const int pos_q = c0 + min(qi, cn - 1);
  const int pos_max = c0 + min(i0 + 15, cn - 1);
  // Q^T operand parts: query r, dims 32c + 8qg .. +7
  u4 qp[3][NKC];
  {
    const float* q = QKV + (size_t)min(qi, cn - 1) * slots * HD + (size_t)h * HD;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      uint32_t pr[3][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t pt[3];
        split3(q[32 * c + 8 * qg + e], pt);
        pr[0][e] = pt[0];
        pr[1][e] = pt[1];
        pr[2][e] = pt[2];
      }
#pragma unroll
      for (int k = 0; k < 3; ++k)
        qp[k][c] = u4{pr[k][0] | (pr[k][1] << 16), pr[k][2] | (pr[k][3] << 16), pr[k][4] | (pr[k][5] << 16),
                      pr[k][6] | (pr[k][7] << 16)};
    }
  }
  const size_t plane = kv_plane(p, HD);
  const uint16_t* kc = p.kv + ((size_t)(l * 2 + 0) * nkv + g) * plane;
  const uint16_t* vc = p.kv + ((size_t)(l * 2 + 1) * nkv + g) * plane;
  f4v acc[NVC];
#pragma unroll
  for (int c = 0; c < NVC; ++c) acc[c] = f4v{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  const int nkb = pos_max / 16 + 1;
  for (int kb = w; kb < nkb; kb += 4) {
    const int j0 = 16 * kb;
    f4v d = {0.f, 0.f, 0.f, 0.f};
    const u4* kr = reinterpret_cast<const u4*>(kc + (size_t)min(j0 + r, pos_max) * HD + 8 * qg);
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      const bf8v ka = __builtin_bit_cast(bf8v, kr[4 * c]);
#pragma unroll
      for (int k = 0; k < 3; ++k) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, __builtin_bit_cast(bf8v, qp[k][c]), d, 0, 0, 0);
    }
    float sc[4];
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + 4 * qg + i;
      sc[i] = qv && j <= pos_q ? d[i] : -INFINITY;
      bm = fmaxf(bm, sc[i]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m, bm);
    const float scale = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    lsum *= scale;
#pragma unroll
    for (int c = 0; c < NVC; ++c) acc[c] *= scale;
    uint32_t pp3[3][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = sc[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[i] - mn);
      lsum += pv;
      uint32_t pt[3];
      split3(pv, pt);
      pp3[0][i] = pt[0];
      pp3[1][i] = pt[1];
      pp3[2][i] = pt[2];
    }
    const int t = min((j0 >> 2) + qg, pos_max >> 2);
#pragma unroll
    for (int c = 0; c < NVC; ++c) {
      const u2 va = *reinterpret_cast<const u2*>(vc + ((size_t)t * HD + 16 * c + r) * 4);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const u2 pb = {pp3[k][0] | (pp3[k][1] << 16), pp3[k][2] | (pp3[k][3] << 16)};
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4v, va), __builtin_bit_cast(s4v, pb),
                                                           acc[c], 0, 0, 0);
      }
    }
  }
  // the query's sum over the four lane groups
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (qg == 0) {
    sm[w][r] = m;
    sl[w][r] = lsum;
  }
  // acc: lane l holds O^T rows (dims) 16c + 4(l/16) + i of column (query) l%16
#pragma unroll
  for (int c = 0; c < NVC; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) so[w][r][16 * c + 4 * qg + i] = acc[c][i];
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * HD; e += 256) {
    const int qr = e / HD, dd = e % HD;
    if (i0 + qr >= cn) continue;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) M = fmaxf(M, sm[v][qr]);
    float L = 0.f, acc_o = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float wgt = sm[v][qr] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[v][qr] - M);
      L = fmaf(sl[v][qr], wgt, L);
      acc_o = fmaf(so[v][qr][dd], wgt, acc_o);
    }
    O[(size_t)(i0 + qr) * nq * HD + (size_t)h * HD + dd] = (uint16_t)f32_to_bf16(acc_o / L);
  }
}

// ---------------------------------------------------------------- LM head
// The last position's final RMSNorm (bf16) against every vocabulary row;
// each wave keeps its best (value, lowest index); logits optional.
__global__ __launch_bounds__(256) void pf_lm_head(const Params* pp, const float* x, float* logits, float* best_v,
                                                  int32_t* best_i) {
  const Params& p = *pp;
  __shared__ float xn[4096];
  __shared__ float red[4];
  const int H = p.H, ln = lane(), w = wave();
  float ss = 0.f;
  for (int e = threadIdx.x; e < H; e += 256) ss += x[e] * x[e];
  ss = wsum(ss);
  if (ln == 0) red[w] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)H + p.eps);
  const __amdgpu_buffer_rsrc_t rw = arena(p);
  for (int e = threadIdx.x; e < H; e += 256) xn[e] = bf16_to_f32((uint16_t)f32_to_bf16(gain(rw, p.final_norm, e) * (x[e] * r)));
  __syncthreads();
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  const int nw = gridDim.x * 4;
  const bool f8 = p.embed.fmt != FMT_BF16;
  // 16-byte loads: 16 FP8 codes or 8 bf16 weights per lane and load, and a
  // wave's consecutive lanes cover consecutive bytes of a row; R rows in
  // flight per wave.  Other row widths take the per-element loop below.
  if (H % (f8 ? 1024 : 512) == 0) {
    constexpr int R = 8;
    const int epl = f8 ? 16 : 8, nk = H / (64 * epl);
    for (int row0 = (blockIdx.x * 4 + w) * R; row0 < p.V; row0 += nw * R) {
      float d[R];
#pragma unroll
      for (int rr = 0; rr < R; ++rr) d[rr] = 0.f;
      for (int k = 0; k < nk; ++k) {
        const int e0 = epl * (ln + 64 * k);
        u4 c[R];
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          const uint64_t row = (uint64_t)min(row0 + rr, p.V - 1);
          const uint64_t off = p.embed.codes + (f8 ? row * H + e0 : 2 * (row * H + e0));
          c[rr] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rw, (uint32_t)off, 0, 0));
        }
        if (f8) {
          float xv[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) xv[j] = xn[e0 + j];
#pragma unroll
          for (int rr = 0; rr < R; ++rr) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float wv[4];
              e4m3x4_to_f32(c[rr][q], wv);
#pragma unroll
              for (int j = 0; j < 4; ++j) d[rr] = fmaf(xv[4 * q + j], wv[j], d[rr]);
            }
          }
        } else {
          float xv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) xv[j] = xn[e0 + j];
#pragma unroll
          for (int rr = 0; rr < R; ++rr) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              d[rr] = fmaf(xv[2 * q], bf16_lo(c[rr][q]), d[rr]);
              d[rr] = fmaf(xv[2 * q + 1], bf16_hi(c[rr][q]), d[rr]);
            }
          }
        }
      }
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const int row = row0 + rr;
        float v = wsum(d[rr]);
        if (f8)
          v *= __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rw, (uint32_t)(p.embed.scales + 4ull * min(row, p.V - 1)), 0, 0));
        if (row < p.V) {
          if (logits && ln == 0) logits[row] = v;
          if (v > bv) {   // rows ascend: a tie keeps the lower index
            bv = v;
            bi = row;
          }
        }
      }
    }
    if (ln == 0) {
      best_v[blockIdx.x * 4 + w] = bv;
      best_i[blockIdx.x * 4 + w] = bi;
    }
    return;
  }
  for (int row = blockIdx.x * 4 + w; row < p.V; row += nw) {
    float d = 0.f;
    if (p.embed.fmt == FMT_BF16) {
      for (int e = ln; e < H; e += 64) d = fmaf(xn[e], gain(rw, p.embed.codes + 2ull * row * H, e), d);
      d = wsum(d);
    } else {
      for (int e = ln; e < H; e += 64) {
        const uint32_t c = __builtin_amdgcn_raw_buffer_load_b8(rw, (uint32_t)(p.embed.codes + (uint64_t)row * H + e), 0, 0);
        d = fmaf(xn[e], e4m3_to_f32(c), d);
      }
      d = wsum(d) * __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, (uint32_t)(p.embed.scales + 4ull * row), 0, 0));
    }
    if (logits && ln == 0) logits[row] = d;
    if (d > bv) {   // rows ascend: a tie keeps the lower index
      bv = d;
      bi = row;
    }
  }
  if (ln == 0) {
    best_v[blockIdx.x * 4 + w] = bv;
    best_i[blockIdx.x * 4 + w] = bi;
  }
}

// One wave: each lane scans every 64th entry, then a butterfly over the
// lanes; the larger value wins, and on equal values the lower index.
__global__ void pf_argmax(const float* best_v, const int32_t* best_i, int n, int32_t* out) {
  if (blockIdx.x != 0 || threadIdx.x >= 64) return;
  const int ln = threadIdx.x;
  float b = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int k = ln; k < n; k += 64) {
    const float v = best_v[k];
    const int i = best_i[k];
    if (v > b || (v == b && i < bi)) {
      b = v;
      bi = i;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float v = __shfl_xor(b, off);
    const int i = __shfl_xor(bi, off);
    if (v > b || (v == b && i < bi)) {
      b = v;
      bi = i;
    }
  }
  if (ln == 0) *out = bi;
}

// The split-K partials added into the residual rows, fused with the next
// RMSNorm: one workgroup per row of H <= 4096, each thread keeping its
// elements (e = thread + 256k) in registers.  The sums, the sum of squares
// and the scaling take the same order as pf_add_partials then pf_rmsnorm.
__global__ __launch_bounds__(256) void pf_add_partials_norm(const Params* pp, const float* P, int nz, int H, size_t n,
                                                            float* X, uint64_t g_off, uint16_t* A) {
  const Params& p = *pp;
  __shared__ float red[4];
  const int i = blockIdx.x;
  float xr[16];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = threadIdx.x + 256 * k;
    if (e < H) {
      const size_t j = (size_t)i * H + e;
      float v = P[j];
      for (int z = 1; z < nz; ++z) v += P[(size_t)z * n + j];
      const float x = X[j] + v;
      X[j] = x;
      xr[k] = x;
      ss += x * x;
    }
  }
  ss = wsum(ss);
  if (lane() == 0) red[wave()] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float r = 1.0f / sqrtf(tot / (float)H + p.eps);
  const __amdgpu_buffer_rsrc_t rw = arena(p);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = threadIdx.x + 256 * k;
    if (e < H) A[(size_t)i * H + e] = (uint16_t)f32_to_bf16(gain(rw, g_off, e) * (xr[k] * r));
  }
}

// X[i] += P[0][i] + P[1][i] + ... (the split-K partials, in order)
__global__ __launch_bounds__(256) void pf_add_partials(const float* P, int nz, size_t n, float* X) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    float v = P[i];
    for (int z = 1; z < nz; ++z) v += P[(size_t)z * n + i];
    X[i] += v;
  }
}

template <int EPI, int T>
hipError_t gemm_t(uint32_t fmt, const Params* pp, const Mat* mat, int N, uint64_t lo, const uint16_t* A, int M, float* C,
                  uint16_t* Hout, hipStream_t s, int nz = 1) {
  const dim3 grid((N + T - 1) / T, (M + T - 1) / T, nz);
  if (fmt == FMT_BF16) hipLaunchKernelGGL((pf_gemm<FMT_BF16, EPI, T>), grid, dim3(256), 0, s, pp, mat, lo, A, M, C, Hout);
  else if (fmt == FMT_FP8) hipLaunchKernelGGL((pf_gemm<FMT_FP8, EPI, T>), grid, dim3(256), 0, s, pp, mat, lo, A, M, C, Hout);
  else hipLaunchKernelGGL((pf_gemm<FMT_FP4, EPI, T>), grid, dim3(256), 0, s, pp, mat, lo, A, M, C, Hout);
  return hipGetLastError();
}
// 64 x 64 tiles where they give at least one workgroup per compute unit, else
// 32 x 32
template <int EPI>
hipError_t gemm(uint32_t fmt, const Params* pp, const Mat* mat, int N, uint64_t lo, const uint16_t* A, int M, float* C,
                uint16_t* Hout, hipStream_t s) {
  if ((long)((N + 127) / 128) * ((M + 127) / 128) >= 256) return gemm_t<EPI, 128>(fmt, pp, mat, N, lo, A, M, C, Hout, s);
  if ((long)((N + 63) / 64) * ((M + 63) / 64) >= 256) return gemm_t<EPI, 64>(fmt, pp, mat, N, lo, A, M, C, Hout, s);
  return gemm_t<EPI, 32>(fmt, pp, mat, N, lo, A, M, C, Hout, s);
}
template <int T>
hipError_t gemm_resid_t(uint32_t fmt, const Params* pp, const Mat* mat, int N, int K, uint64_t lo, const uint16_t* A,
                        int M, float* X, float* ws, size_t ws_floats, uint64_t g_off, uint16_t* An, hipStream_t s) {
  const long tiles = (long)((N + T - 1) / T) * ((M + T - 1) / T);
  int nz = 1;
  while (nz < 4 && tiles * nz * 2 <= 512 && (K / (2 * nz)) % (2 * BK) == 0 && (size_t)2 * nz * M * N <= ws_floats) nz *= 2;
  if (nz == 1) {
    hipError_t e = gemm_t<EPI_RESID, T>(fmt, pp, mat, N, lo, A, M, X, nullptr, s);
    if (e != hipSuccess || !An) return e;
    hipLaunchKernelGGL(pf_rmsnorm, dim3(M), dim3(256), 0, s, pp, X, M, N, g_off, An);
    return hipGetLastError();
  }
  hipError_t e = gemm_t<EPI_PARTIAL, T>(fmt, pp, mat, N, lo, A, M, ws, nullptr, s, nz);
  if (e != hipSuccess) return e;
  const size_t n = (size_t)M * N;
  if (An)
    hipLaunchKernelGGL(pf_add_partials_norm, dim3(M), dim3(256), 0, s, pp, ws, nz, N, n, X, g_off, An);
  else
    hipLaunchKernelGGL(pf_add_partials, dim3((unsigned)std::min<size_t>((n + 255) / 256, 1024)), dim3(256), 0, s, ws,
                       nz, n, X);
  return hipGetLastError();
}
// A product added into the residual X [M x N].  Where the tiles give fewer
// than two workgroups per compute unit, K is split over nz workgroups
// (nz <= 4, partials in `ws`, which holds ws_floats) and the partials are
// added in a fixed order.
// 128 x 128 tiles once four K slices of them fill the device, else 64 x 64.
// With An, the RMSNorm of the new residual (gains at g_off) follows into An,
// fused with the partials' sum where K is split.
hipError_t gemm_resid(uint32_t fmt, const Params* pp, const Mat* mat, int N, int K, uint64_t lo, const uint16_t* A, int M,
                      float* X, float* ws, size_t ws_floats, uint64_t g_off, uint16_t* An, hipStream_t s) {
  if ((long)((N + 127) / 128) * ((M + 127) / 128) * 4 >= 256 && (K / 4) % (2 * BK) == 0 &&
      (size_t)4 * M * N <= ws_floats)
    return gemm_resid_t<128>(fmt, pp, mat, N, K, lo, A, M, X, ws, ws_floats, g_off, An, s);
  return gemm_resid_t<64>(fmt, pp, mat, N, K, lo, A, M, X, ws, ws_floats, g_off, An, s);
}

}  // namespace

hipError_t launch_prefill_chunk(const PrefillArgs& a, hipStream_t s) {
  const Params* pp = a.params;
  const int cn = a.cn, H = a.H, hd = a.hd, nq = a.nq, nkv = a.nkv, I = a.I;
  const int nqkv = (nq + 2 * nkv) * hd;
  hipLaunchKernelGGL(pf_embed, dim3(cn), dim3(256), 0, s, pp, a.tokens, cn, a.X);
  for (int l = 0; l < a.L; ++l) {
    const uint64_t lo = (uint64_t)l * a.layer_stride;
    // later layers' input norms come with the previous layer's down product
    if (l == 0) hipLaunchKernelGGL(pf_rmsnorm, dim3(cn), dim3(256), 0, s, pp, a.X, cn, H, a.in_norm + lo, a.A);
    hipError_t e = gemm<EPI_STORE>(a.fmt_lin, pp, a.mat_qkv, nqkv, lo, a.A, cn, a.QKV, nullptr, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pf_qkv_post, dim3((cn * (nq + 2 * nkv) + 3) / 4), dim3(256), 0, s, pp, l, a.c0, cn, a.QKV);
    const dim3 ga(((cn + 15) / 16) * nq);
    if (hd == 128)
      hipLaunchKernelGGL(pf_attention_mc<128>, ga, dim3(256), 0, s, pp, l, a.c0, cn, a.QKV, a.A);
    else if (hd == 64)
      hipLaunchKernelGGL(pf_attention_mc<64>, ga, dim3(256), 0, s, pp, l, a.c0, cn, a.QKV, a.A);
    else
      return hipErrorInvalidValue;
    // the QKV outputs are used up: their buffer holds the split-K partials
    const size_t ws = (size_t)kPrefillChunk * nqkv;
    e = gemm_resid(a.fmt_lin, pp, a.mat_o, H, nq * hd, lo, a.A, cn, a.X, a.QKV, ws, a.post_norm + lo, a.A, s);
    if (e != hipSuccess) return e;
    e = gemm<EPI_SWIGLU>(a.fmt_lin, pp, a.mat_gu, 2 * I, lo, a.A, cn, nullptr, a.Hb, s);
    if (e != hipSuccess) return e;
    const bool next = l + 1 < a.L;
    e = gemm_resid(a.fmt_down, pp, a.mat_down, H, I, lo, a.Hb, cn, a.X, a.QKV, ws,
                   next ? a.in_norm + lo + a.layer_stride : 0, next ? a.A : nullptr, s);
    if (e != hipSuccess) return e;
  }
  if (a.last) {
    hipLaunchKernelGGL(pf_lm_head, dim3(kPrefillHeadGroups), dim3(256), 0, s, pp, a.X + (size_t)(cn - 1) * H, a.logits,
                       a.best_v, a.best_i);
    hipLaunchKernelGGL(pf_argmax, dim3(1), dim3(64), 0, s, a.best_v, a.best_i, kPrefillHeadGroups * 4, a.next);
  }
  return hipGetLastError();
}

}  // namespace mk
