// Structures shared by the host launcher and the gfx950 kernels.
#pragma once
#include <stdint.h>

// Device code sees the buffers through address-space-1 (global) pointers, so
// the compiler emits global_* instead of flat_* accesses: flat loads count
// against the LDS counter too, and waiting on LDS would then also drain the
// weight prefetch.  The host pass sees plain pointers of the same size.
#if defined(__HIP_DEVICE_COMPILE__)
#define MK_GLOBAL __attribute__((address_space(1)))
#else
#define MK_GLOBAL
#endif
#define GCAST(T, ptr) reinterpret_cast<MK_GLOBAL T*>(ptr)

namespace mk {

enum : uint32_t { FMT_BF16 = 0, FMT_FP8 = 1, FMT_FP4 = 2 };

constexpr int kThreads = 512;            // threads per workgroup (8 wave64s)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxOwn = 64;              // residual rows one workgroup may own
constexpr int kMaxVecWords = 6144;       // words one gather may bring into LDS
constexpr int kMaxPart = 2048;           // GEMV (row, 1024-chunk) items per workgroup per phase
constexpr int kPhaseBits = 10;           // low bits of an exchange tag hold the phase id
constexpr uint32_t kEpochMask = (1u << (32 - kPhaseBits)) - 1;

// One packed matrix in the weight arena (byte offsets from the arena base).
//  bf16: codes = N*K uint16.  fp8: codes = N*K bytes, scales = N fp32.
//  fp4 : codes = N*K/2 bytes (element 2j in the low nibble of byte j),
//        scales = N*K/16 E4M3 block scales, tscale = up to 3 fp32 tensor scales.
struct Mat {
  uint64_t codes, scales, tscale;
  uint32_t N, K;
  uint32_t fmt;
  uint32_t ts_mode;   // fp4 tensor-scale index per row: 0 single; 1 row<b0 ? 0 : row<b1 ? 1 : 2; 2 row&1
  uint32_t ts_b0, ts_b1;
};

// Matrices of one layer.  qkv = [q; k; v] rows; gu = gate and up rows
// interleaved (row 2i gate_i, row 2i+1 up_i).  Norm gains are bf16 arrays.
struct Layer {
  Mat qkv, o, gu, down;
  uint64_t in_norm, post_norm, q_norm, k_norm;
};

// Exchange buffers in scratch, in 64-bit words.  Every word is
// (payload << 32) | tag, written and read with agent-scope atomic stores and
// loads.  Buffers a consumer set reads are replicated R times; layer-indexed
// buffers alternate between two parities.
struct Xch {
  uint64_t x_d, x_o, qkv, o, h;   // replicated vectors: base word offsets
  uint64_t rep_x, rep_qkv, rep_o, rep_h;  // stride between replicas (words)
  uint64_t par_x, par_qkv, par_o, par_h;  // stride between parities (words)
  uint64_t part, par_part;        // split-attention partials [ns_max][nq][hd+2]
  uint64_t arg;                   // argmax slots [grid][2]
  uint64_t err;                   // error word (uint32 in a 64-bit slot)
  uint64_t amax;                  // packing scratch: tensor abs-max (uint32 bits)
  uint64_t words;                 // total words
};

struct Params {
  MK_GLOBAL const uint8_t* w;   // weight arena
  MK_GLOBAL uint16_t* kv;       // [L][2][nkv][max_ctx][hd] bf16
  MK_GLOBAL const float* rope;  // [max_ctx][hd/2][2] cos, sin
  MK_GLOBAL uint64_t* xch;      // scratch
  void* trace;                  // mk_trace_rec records, or null
  int L, H, nq, nkv, hd, I, V, max_ctx;
  float eps;
  Mat embed;
  Layer layer0;
  uint64_t layer_stride;  // bytes between consecutive layers' matrices
  uint64_t final_norm;
  Xch x;
  int grid, R, att_target, ns_max;
  uint64_t spin_limit;    // s_memrealtime ticks
  uint32_t tag_skew;      // test hook: added to every expected tag (non-zero makes every wait time out)
  uint32_t poll_sleep;    // s_sleep units (64 clocks each) between polls of a word that is not ready
  int n_phases;           // phase ids per step (trace stride per workgroup)
};

}  // namespace mk
