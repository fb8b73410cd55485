// Inter-workgroup exchange and the courier / compute hand-off inside a
// workgroup, for the persistent decode kernel.
//
// The monolith page ("Design decisions", the sync experiments) replaces
// grid-wide barriers by per-tile counters with release/acquire ordering, so a
// consumer waits only for the tiles it reads.  On gfx950 the eight XCDs have
// separate L2 caches, and an agent-scope release/acquire pair costs an L2
// write-back plus an L2 invalidate (the invalidate would also drop the
// prefetched weights).  Here instead every produced value travels in its own
// 64-bit word, (payload << 32) | tag, stored with an agent-scope relaxed
// atomic store (coherent across XCDs without cache maintenance).  The tag is
// (epoch << 10) | vector id, unique per launch and vector, so a word that
// carries the expected tag holds that producer's value: flag and data are one
// atomic object and no fence is needed.
//
// gfx9 retires a wave's vector memory operations in order under one counter
// (vmcnt), so a poll issued behind a weight prefetch would return only after
// the prefetch.  Only the courier wave of a workgroup polls; it keeps no
// weight loads in flight.  It reads two words per lane per 16-byte load
// (each 8-byte half is one producer's atomic store and carries its own tag),
// re-polls only what is missing, and once a vector is complete it writes the
// payloads (normalised where the consumer wants that) into LDS and bumps the
// workgroup's LDS sequence counter.  Compute waves wait on that counter with
// LDS reads, which count against lgkmcnt, not vmcnt.
//
// Each courier wait is bounded: past `spin_limit` s_memrealtime ticks, or once
// any workgroup has recorded an error, it gives up and raises the abort value
// in the sequence counter, which ends the compute waves' waits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_shared.h"

namespace mk {

enum : uint32_t { ERR_TIMEOUT = 1u, ERR_TOKEN = 2u };

#ifdef MK_STRESS
// Stress build, the race-detection stand-in: a pseudo-random pause of 0 to
// 31 x 2 s_sleep units (up to about 1.7 us) before every exchange store and
// every courier hand-over.  The pause depends on the clock, the workgroup,
// the wave and the store site, so every run interleaves the producers,
// the consumers' poll rounds and the LDS hand-offs differently.  A missing
// wait or a value read before it is complete would show as a changed
// result; the results must stay bit-identical to the headline build's.
__device__ __forceinline__ void stress_pause(uint32_t site) {
  uint32_t h = site ^ (uint32_t)__builtin_amdgcn_s_memrealtime() ^ (blockIdx.x * 0x9E3779B1u) ^
               ((threadIdx.x >> 6) * 0x85EBCA77u);
  h ^= h >> 16;
  h *= 0x7FEB352Du;
  h ^= h >> 15;
  h *= 0x846CA68Bu;
  h ^= h >> 16;
  const uint32_t n = __builtin_amdgcn_readfirstlane(h) & 31u;
  for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(2);
}
#endif
constexpr uint32_t kAbort = 0xFFFFFFFFu;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void st_word(MK_GLOBAL uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_word(MK_GLOBAL uint64_t* p, uint32_t payload, uint32_t tag) {
  st_word(p, ((uint64_t)payload << 32) | tag);
}
__device__ __forceinline__ uint32_t make_tag(uint32_t epoch, uint32_t id) { return (epoch << kPhaseBits) | id; }
__device__ __forceinline__ uint32_t vec_id(int l, int type) { return (uint32_t)(2 + kTypes * l + type); }

__device__ __forceinline__ MK_GLOBAL uint32_t* err_word(const Params& p) {
  return GCAST(uint32_t, p.xch + p.x.err);
}
__device__ __forceinline__ void raise_error(const Params& p, uint32_t code) {
  __hip_atomic_fetch_or(err_word(p), code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exchange vector `type` of layer l: pointer, and word offset in the scratch buffer.
__device__ __forceinline__ MK_GLOBAL uint64_t* xvec(const Params& p, int l, int type) {
  return p.xch + p.x.base + (uint64_t)l * p.x.layer_words + p.x.off[type];
}
__device__ __forceinline__ uint32_t xword(const Params& p, int l, int type) {
  return (uint32_t)(p.x.base + (uint64_t)l * p.x.layer_words + p.x.off[type]);
}

// Wait until this wave's LDS accesses have completed, without waiting for
// its global loads (s_waitcnt lgkmcnt(0); vmcnt and expcnt at their maxima),
// and keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_drain() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ uint32_t lds_ld(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Workgroup barrier that waits only for LDS (the waves may keep global loads
// in flight across it).
__device__ __forceinline__ void lds_barrier() {
  lds_drain();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Compute waves: wait until the courier has handed over `want` inputs.
// Returns false if the courier aborted, or (a safety net: the courier's own
// waits are bounded) after `spin_limit` ticks.  The loop polls LDS without
// sleeping between reads: a sleep of 64 clocks between polls cost 0.8 % of
// the step (five hand-offs per layer).
__device__ __forceinline__ bool wait_seq(const Params& p, const uint32_t* seq, uint32_t want) {
  uint32_t s = __builtin_amdgcn_readfirstlane(lds_ld(seq));
  if (s >= want) return s != kAbort;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t n = 1;; ++n) {
    s = __builtin_amdgcn_readfirstlane(lds_ld(seq));
    if (s >= want) return s != kAbort;
    if ((n & 255u) == 0 && __builtin_amdgcn_s_memrealtime() - t0 > p.spin_limit) {
      if ((threadIdx.x & 63) == 0) raise_error(p, ERR_TIMEOUT);
      return false;
    }
  }
}

// Courier: publish one more input (LDS writes first, then the counter).
__device__ __forceinline__ void hand_over(uint32_t* seq, uint32_t value) {
#ifdef MK_STRESS
  stress_pause(value * 0x27D4EB2Fu);
#endif
  lds_drain();
  if ((threadIdx.x & 63) == 0) lds_st(seq, value);
  lds_drain();
}

// 16-byte load of two consecutive exchange words with device-scope
// coherence (sc1), through a buffer resource over the scratch buffer.  Each
// 8-byte half is checked against the tag on its own, so what this relies on
// is that the memory system never splits an aligned 8-byte word: a half is
// seen either before or after its producer's single 8-byte store, never
// half-written.  The two halves may come from different moments (they are
// two producers' words, or one word seen before it was written), which the
// per-half tag check absorbs.  The 16-byte load is not assumed to be atomic
// as a whole.
__device__ __forceinline__ v4u ld_pair(__amdgpu_buffer_rsrc_t r, uint32_t word) {
  return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, word * 8u, 0, 16));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t xch_rsrc(const Params& p) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p.xch, (short)0, (int)(p.x.words * 8), 0x00020000);
}

// Store one exchange word, device-scope coherent (sc1), through the scratch
// buffer resource.  A byte offset past the buffer (see kOOB) drops the
// store, which lets a wave skip a store without a branch.
__device__ __forceinline__ void st_xword(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint32_t payload,
                                         uint32_t tag) {
#ifdef MK_STRESS
  stress_pause(__builtin_amdgcn_readfirstlane(byte_off) ^ tag);
#endif
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v2u{tag, payload}), r, byte_off, 0, 16);
}

// Gather `npairs` (>= 1) pairs of words; pair j is at word src(j) (even,
// the two words consecutive).  Lane l owns pairs j0 + l + jstep*k, k < MAXK;
// their payloads land in lo[k] (word 2j) and hi[k] (word 2j+1).  Each round
// issues every missing pair's load before waiting, so one round costs one
// memory latency.  Returns false on timeout or when another workgroup has
// failed.  The courier gathers with j0 = 0, jstep = 64; the waves of a
// workgroup with no loads in flight may share a gather with other strides.
template <int MAXK, class F>
__device__ __forceinline__ bool gather_pairs(const Params& p, __amdgpu_buffer_rsrc_t r, int npairs, uint32_t tag,
                                             uint32_t (&lo)[MAXK], uint32_t (&hi)[MAXK], F src, int j0 = 0,
                                             int jstep = 64) {
  const int lane = threadIdx.x & 63;
  tag += p.tag_skew;
  uint32_t pend = 0;
  v4u v[MAXK];
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    const int j = j0 + lane + jstep * k;
    if (j < npairs) pend |= 1u << k;
    v[k] = ld_pair(r, src(min(j, npairs - 1)));   // clamped: no load behind a branch
  }
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  uint32_t rounds = 0;
  while (true) {
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      if (v[k].x == tag && v[k].z == tag) pend &= ~(1u << k);
      lo[k] = v[k].y;
      hi[k] = v[k].w;
    }
    if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) return true;
    ++rounds;
    if (__builtin_amdgcn_s_memrealtime() - t0 > p.spin_limit) {
      raise_error(p, ERR_TIMEOUT);
      return false;
    }
    if ((rounds & 63u) == 0 &&
        __hip_atomic_load(err_word(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
      return false;
    for (uint32_t z = 0; z < p.poll_sleep; ++z) __builtin_amdgcn_s_sleep(8);   // back-off: ~512 clocks each
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < MAXK; ++k)
      if ((pend >> k) & 1u) v[k] = ld_pair(r, src(j0 + lane + jstep * k));
  }
}

// Courier gather of a vector in the per-producer layout: the lane's pair k
// (pair lane + 64k of the vector, valid if below npairs) is at word
// base + off[k]; off[] was computed once per launch (clamped for lanes past
// the end).
template <int MAXK>
__device__ __forceinline__ bool gather_pairs_at(const Params& p, __amdgpu_buffer_rsrc_t r, int npairs, uint32_t tag,
                                                uint32_t (&lo)[MAXK], uint32_t (&hi)[MAXK], uint32_t base,
                                                const uint32_t (&off)[MAXK]) {
  const int lane = threadIdx.x & 63;
  tag += p.tag_skew;
  uint32_t pend = 0;
  v4u v[MAXK];
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    if (lane + 64 * k < npairs) pend |= 1u << k;
    v[k] = ld_pair(r, base + off[k]);
  }
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  uint32_t rounds = 0;
  while (true) {
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      if (v[k].x == tag && v[k].z == tag) pend &= ~(1u << k);
      lo[k] = v[k].y;
      hi[k] = v[k].w;
    }
    if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) return true;
    ++rounds;
    if (__builtin_amdgcn_s_memrealtime() - t0 > p.spin_limit) {
      raise_error(p, ERR_TIMEOUT);
      return false;
    }
    if ((rounds & 63u) == 0 &&
        __hip_atomic_load(err_word(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
      return false;
    for (uint32_t z = 0; z < p.poll_sleep; ++z) __builtin_amdgcn_s_sleep(8);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < MAXK; ++k)
      if ((pend >> k) & 1u) v[k] = ld_pair(r, base + off[k]);
  }
}

// The same gather, but each pair's payloads are handed to put(j, lo, hi)
// (an LDS write) as soon as the pair carries the tag, so a lane keeps only
// its loads in flight in registers.
template <int MAXK, class F, class G>
__device__ __forceinline__ bool gather_pairs_to(const Params& p, __amdgpu_buffer_rsrc_t r, int npairs, uint32_t tag,
                                                F src, G put, int j0, int jstep) {
  const int lane = threadIdx.x & 63;
  tag += p.tag_skew;
  uint32_t pend = 0;
  v4u v[MAXK];
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    const int j = j0 + lane + jstep * k;
    if (j < npairs) pend |= 1u << k;
    v[k] = ld_pair(r, src(min(j, npairs - 1)));
  }
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  uint32_t rounds = 0;
  while (true) {
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
      if (((pend >> k) & 1u) && v[k].x == tag && v[k].z == tag) {
        pend &= ~(1u << k);
        put(j0 + lane + jstep * k, v[k].y, v[k].w);
      }
    }
    if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) return true;
    ++rounds;
    if (__builtin_amdgcn_s_memrealtime() - t0 > p.spin_limit) {
      raise_error(p, ERR_TIMEOUT);
      return false;
    }
    if ((rounds & 63u) == 0 &&
        __hip_atomic_load(err_word(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
      return false;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < MAXK; ++k)
      if ((pend >> k) & 1u) v[k] = ld_pair(r, src(j0 + lane + jstep * k));
  }
}

}  // namespace mk
