// Inter-workgroup exchange for the persistent decode kernel.
//
// The monolith page ("Design decisions", sync experiments) replaces grid-wide
// barriers by per-tile counters with release/acquire ordering, so that a
// consumer waits only for the tiles it reads.  On gfx950 the eight XCDs have
// separate L2 caches, and an agent-scope release/acquire pair costs an L2
// write-back plus an L2 invalidate.  Measured on MI355X, counters with those
// fences take 16-21 us per all-to-all round of 256 workgroups, against
// 2.2-5 us for the scheme used here:
//
//   * every produced value travels in its own 64-bit word,
//     (payload << 32) | tag, written with an agent-scope relaxed atomic
//     store and read with an agent-scope relaxed atomic load (the compiler
//     emits sc1 accesses, coherent across XCDs without cache maintenance);
//   * the tag is (epoch << 10) | phase, unique per launch and phase, so a
//     consumer that reads a word carrying the expected tag holds that
//     producer's value: the flag and the data are one atomic object, and no
//     fence is needed;
//   * producers write R replicas of each word and consumer workgroup b reads
//     replica b % R, which spreads the consumers' polling over memory
//     channels instead of one hot spot.
//
// Each wait is bounded: past `spin_limit` s_memrealtime ticks, or once any
// workgroup has recorded an error, the wait gives up and the kernel exits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_shared.h"

namespace mk {

enum : uint32_t { ERR_TIMEOUT = 1u, ERR_TOKEN = 2u };

__device__ __forceinline__ uint64_t ld_word(MK_GLOBAL const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(MK_GLOBAL uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t make_tag(uint32_t epoch, uint32_t phase) {
  return (epoch << kPhaseBits) | phase;
}

__device__ __forceinline__ MK_GLOBAL uint32_t* err_word(const Params& p) {
  return GCAST(uint32_t, p.xch + p.x.err);
}
__device__ __forceinline__ void raise_error(const Params& p, uint32_t code) {
  __hip_atomic_fetch_or(err_word(p), code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Write word i of a replicated vector: one copy per replica.
__device__ __forceinline__ void publish(MK_GLOBAL uint64_t* base, uint64_t rep_stride, int R, int i,
                                        uint32_t payload, uint32_t tag) {
  const uint64_t v = ((uint64_t)payload << 32) | tag;
  for (int r = 0; r < R; ++r) st_word(base + (uint64_t)r * rep_stride + i, v);
}

// Poll one word until its tag matches; false on timeout or a recorded error.
__device__ __forceinline__ bool wait_word(MK_GLOBAL const uint64_t* src, uint32_t tag, uint64_t& v,
                                          const Params& p, uint64_t t0) {
  uint32_t n = 0;
  while ((uint32_t)v != tag) {
    // back off between polls: polling traffic goes to the memory side and
    // slows every other access there
    switch (p.poll_sleep) {
      case 0: break;
      case 1: __builtin_amdgcn_s_sleep(1); break;
      case 2: __builtin_amdgcn_s_sleep(2); break;
      case 3: __builtin_amdgcn_s_sleep(4); break;
      case 4: __builtin_amdgcn_s_sleep(8); break;
      default: __builtin_amdgcn_s_sleep(16); break;
    }
    if ((++n & 63u) == 0) {
      if (__builtin_amdgcn_s_memrealtime() - t0 > p.spin_limit) {
        raise_error(p, ERR_TIMEOUT);
        return false;
      }
      if (__hip_atomic_load(err_word(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
    }
    v = ld_word(src);
  }
  return true;
}

// All threads of the workgroup read words [0, n) of `src` (one replica),
// waiting for each to carry `tag`, and store the payloads to dst[0, n).
// Returns this thread's success; callers combine it across the workgroup.
__device__ __forceinline__ bool gather(MK_GLOBAL const uint64_t* src, int n, uint32_t tag, uint32_t* dst,
                                       const Params& p) {
  constexpr int B = 4;  // words in flight per thread per pass
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  tag += p.tag_skew;
  bool ok = true;
  for (int base = 0; base < n; base += kThreads * B) {
    uint64_t v[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {  // unconditional (clamped) loads: no branch, no early wait
      const int i = base + (int)threadIdx.x + k * kThreads;
      v[k] = ld_word(src + min(i, n - 1));
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int i = base + (int)threadIdx.x + k * kThreads;
      if (i < n && ok) {
        ok = wait_word(src + i, tag, v[k], p, t0);
        dst[i] = (uint32_t)(v[k] >> 32);
      }
    }
  }
  return ok;
}

// The same for words base[idx(i)], i in [0, n), stored to dst[i].
template <class F>
__device__ __forceinline__ bool gather_map(MK_GLOBAL const uint64_t* base, int n, uint32_t tag, uint32_t* dst,
                                           const Params& p, F idx) {
  constexpr int B = 4;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  tag += p.tag_skew;
  bool ok = true;
  for (int b0 = 0; b0 < n; b0 += kThreads * B) {
    uint64_t v[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int i = b0 + (int)threadIdx.x + k * kThreads;
      v[k] = ld_word(base + idx(min(i, n - 1)));
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int i = b0 + (int)threadIdx.x + k * kThreads;
      if (i < n && ok) {
        ok = wait_word(base + idx(i), tag, v[k], p, t0);
        dst[i] = (uint32_t)(v[k] >> 32);
      }
    }
  }
  return ok;
}

}  // namespace mk
