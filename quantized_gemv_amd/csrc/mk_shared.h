// Structures shared by the host launcher and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
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

// A decode workgroup is one courier wave (wave 0) and seven compute waves.
// The courier alone polls the exchange words in global memory; it gathers
// each input vector into LDS and hands it over with an LDS sequence counter.
// The compute waves hold their rows' weights in registers, a full layer
// ahead, and never wait on global memory for anything but their own weights.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCW = kWaves - 1;              // compute waves (wave ids 1..7)
constexpr int kPhaseBits = 10;               // low bits of an exchange tag hold the vector id
constexpr uint32_t kEpochMask = (1u << (32 - kPhaseBits)) - 1;
constexpr int kTypes = 6;                    // exchange vectors per layer (see below)
constexpr int kMaxLayers = (int)((1u << kPhaseBits) - 4) / kTypes;   // 170

// Weights and exchange words are read and written through buffer resources
// (32-bit offsets).  kOOB is an offset past the end of every such buffer: a
// load there returns zeros and a store there is dropped, without touching
// memory, which lets a wave skip a row or a store without a branch.
constexpr uint32_t kOOB = 0x7FFFFFF0u;
constexpr uint64_t kMaxBuffer = 0x7FFF0000ull;   // largest buffer read that way

// Units per compute wave and phase (the host checks its schedule against these).
constexpr int kMaxQKV = 3, kMaxO = 1, kMaxGU = 2, kMaxD = 1;
constexpr int kSchedInts = 32;               // ints per workgroup header and per compute wave

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

// Exchange vectors of layer l (word offsets inside the layer's block).  Each
// word is (payload << 32) | tag with tag = (epoch << kPhaseBits) | vector id,
// vector id = 2 + kTypes*l + type; the argmax words of the step use id
// 2 + kTypes*L.  V_ATT holds the split-attention partials:
// [nkv][split_max][split_pw] words.
enum : int { V_QKV = 0, V_ATT = 1, V_O = 2, V_XO = 3, V_H = 4, V_XD = 5 };
struct Xch {
  uint64_t base;              // word offset of layer 0's block
  uint64_t layer_words;       // words per layer block
  uint64_t off[kTypes];       // offset of each vector in a block
  // Vectors written by many producers (the residuals after O and down, the
  // SwiGLU output) are laid out per producer: the vector's words are dealt
  // in contiguous blocks of even length over pad_c producers, and block i
  // starts a line of its own, at word i * pad_stride (0 = packed layout).
  uint32_t pad_c[kTypes], pad_stride[kTypes];
  uint64_t arg;               // argmax words [grid][2] (value, index)
  uint64_t bar;               // grid-barrier variant: one arrival counter per barrier of a step (5L + 1)
  uint64_t err;               // error word (uint32 in a 64-bit slot)
  uint64_t amax;              // packing scratch: tensor abs-max (uint32 bits)
  uint64_t words;             // total words
};

// Word w of an n-word exchange vector in the per-producer layout (see Xch).
__host__ __device__ inline uint32_t xpad_word(uint32_t w, uint32_t n, uint32_t c, uint32_t stride) {
  if (c == 0) return w;
  const uint32_t np = n / 2, j = w / 2;
  const uint32_t i = ((j + 1) * c - 1) / np;   // the block holding pair j
  return i * stride + 2 * (j - np * i / c) + (w & 1u);
}

// Per-workgroup header of the work table (ints).
enum : int {
  S_FLAGS = 0,      // bit 0: gathers xd (QKV or O units), 1: o, 2: xo (gate/up or down), 3: h
  S_ATT = 1,        // KV head whose attention this workgroup runs (its home workgroup), or -1
  S_NIN = 2,        // inputs the courier gathers per layer
  S_IXD = 3, S_IQKV = 4, S_IO = 5, S_IXO = 6, S_IH = 7,   // input index in the layer, or -1
  // split attention (the kernel variant for long contexts): a GEMV workgroup
  // also takes a slice of one KV head's cached positions, which adds the
  // head's q to its inputs
  S_SPLIT = 8,      // KV head whose positions this workgroup helps with, or -1
  S_SPLIT_IDX = 9,  // its slice index among that head's helpers (1-based; the home takes slice 0)
  S_NIN_L = 10,     // inputs per layer in the split variant
  S_IQS_L = 11, S_IO_L = 12, S_IXO_L = 13, S_IH_L = 14,   // input indices in the split variant, or -1
  kHdrInts = 16,
};
constexpr int kMaxSplit = 32;   // helpers per KV head (the home merges their partials in LDS)
constexpr int kSplitGatherK = 10;   // partial word pairs per lane and round of the home's gather
// Per compute wave: units of each phase (-1 = none), at these offsets, and
// the word each QKV unit stores (the q/k/v vector is laid out per producer
// too: per XCD, the rows of its KV heads are dealt in even blocks over its
// GEMV workgroups, each block starting a 128-byte line).
enum : int { S_QKV = 0, S_O = 4, S_GU = 8, S_D = 12, S_QKVW = 16, kUnitInts = 20 };

struct Params {
  MK_GLOBAL const uint8_t* w;   // weight arena
  uint32_t w_bytes;             // its size (read through a buffer resource: below 2 GB)
  MK_GLOBAL uint16_t* kv;       // per layer K then V, per KV head a plane of ctx4 x hd bf16 (ctx4 = max_ctx
                                // rounded up to 4): K row-major, V in tiles of 4 positions
  MK_GLOBAL const float* rope;  // [max_ctx][hd/2][2] cos, sin
  MK_GLOBAL uint64_t* xch;      // scratch
  void* trace;                  // mk_trace_rec records, or null
  int L, H, nq, nkv, hd, I, V, max_ctx;
  float eps;
  Mat embed;
  Layer layer0;
  uint64_t layer_stride;  // bytes between consecutive layers' matrices
  uint64_t final_norm;
  // Read-only tables in the weight arena (byte offsets), written at bind:
  // the work table (int32, kSchedInts per header and per compute wave) and,
  // right after it, per KV head the word offset (in the q/k/v vector) of
  // each pair of its q rows, k rows and v rows, in that order (int32).
  // Every workgroup reads its rows once per launch.  Being an input of
  // every decode entry point, the arena also serves the step that brings
  // no scratch buffer of its own.
  uint64_t sched, qmap;
  Xch x;
  int grid;
  uint64_t spin_limit;    // s_memrealtime ticks
  uint32_t tag_skew;      // test hook: added to every expected tag (non-zero makes every wait time out)
  uint32_t poll_sleep;    // s_sleep units between courier poll rounds
  int n_phases;           // trace phases per step (trace stride per workgroup)
  int split_max;          // helper slots per KV head in the partials vector
  int split_pw;           // words per helper partial (outputs, maxima, sums; padded)
  uint32_t bar_fence;     // grid-barrier variant: 1 arrive with an agent-scope release and leave with an
                          // agent-scope acquire (L2 write-back and invalidate), 0 relaxed counters
  uint32_t lm_balance;    // several steps per launch: 1 LM-head rows balanced across XCDs, 0 equal shares (default)
};

}  // namespace mk
