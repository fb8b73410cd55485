// X-ray: per-workgroup, per-phase timestamps inside the decode kernel.
//
// The monolith page ("Design decisions", timing; milestone M2) has one lane
// of every block write phase stamps to a preallocated buffer behind a
// compile-time flag, with the SM id, and aligns the clocks offline.  Here
// every stamp is s_memrealtime (a 100 MHz counter common to all XCDs, so no
// alignment is needed).  During the step the stamps live in LDS: the courier
// writes when it began gathering a phase's input, when every word was
// present and when it handed the input over; the compute waves fold in the
// first time one of them saw the input (minimum) and the last time one
// finished its outputs (maximum).  At the end of the step each workgroup
// copies its records, with its HW_ID and XCC_ID registers, to the trace
// buffer.  Without MK_XRAY every macro is empty.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk.h"

namespace mk {

#ifdef MK_XRAY
constexpr int kXrPhases = 6 * 40 + 4;   // X-ray covers models of up to 40 layers
enum : int { XR_START = 0, XR_READY = 1, XR_HANDOFF = 2, XR_SEEN = 3, XR_DONE = 4, XR_M0 = 5 };
struct XrLds {
  unsigned long long v[kXrPhases][8];
};
__device__ __forceinline__ unsigned long long xr_now() { return __builtin_amdgcn_s_memrealtime(); }
#define XR_FIELD XrLds xr;
// every wave clears its share, then the caller's first barrier orders it
#define XR_INIT(s)                                                                   \
  do {                                                                               \
    for (int i_ = threadIdx.x; i_ < kXrPhases * 8; i_ += kThreads)                   \
      (s).xr.v[i_ / 8][i_ % 8] = (i_ % 8) == XR_SEEN ? ~0ull : 0ull;                 \
  } while (0)
#define XR_PUT(s, ph, slot)                                                          \
  do {                                                                               \
    if ((threadIdx.x & 63) == 0 && (ph) < kXrPhases) (s).xr.v[ph][slot] = xr_now();  \
  } while (0)
#define XR_MIN(s, ph, slot)                                                          \
  do {                                                                               \
    if ((threadIdx.x & 63) == 0 && (ph) < kXrPhases) atomicMin(&(s).xr.v[ph][slot], xr_now()); \
  } while (0)
#define XR_MAX(s, ph, slot)                                                          \
  do {                                                                               \
    if ((threadIdx.x & 63) == 0 && (ph) < kXrPhases) atomicMax(&(s).xr.v[ph][slot], xr_now()); \
  } while (0)
// after a workgroup barrier: copy the records out
#define XR_DUMP(s, p)                                                                \
  do {                                                                               \
    if ((p).trace) {                                                                 \
      const uint32_t hw_ = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);      \
      const uint32_t xcc_ = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);     \
      for (int ph_ = threadIdx.x; ph_ < (p).n_phases && ph_ < kXrPhases; ph_ += kThreads) { \
        mk_trace_rec r_;                                                             \
        r_.phase = ph_;                                                              \
        r_.wg = blockIdx.x;                                                          \
        r_.hw_id = hw_;                                                              \
        r_.xcc = xcc_;                                                               \
        r_.active = (s).xr.v[ph_][XR_START] != 0 || (s).xr.v[ph_][XR_DONE] != 0;     \
        r_.pad = 0;                                                                  \
        r_.t_start = (s).xr.v[ph_][XR_START];                                        \
        r_.t_ready = (s).xr.v[ph_][XR_READY];                                        \
        r_.t_handoff = (s).xr.v[ph_][XR_HANDOFF];                                    \
        r_.t_seen = (s).xr.v[ph_][XR_SEEN] == ~0ull ? 0 : (s).xr.v[ph_][XR_SEEN];    \
        r_.t_done = (s).xr.v[ph_][XR_DONE];                                          \
        for (int k_ = 0; k_ < 3; ++k_) r_.t_mark[k_] = (s).xr.v[ph_][XR_M0 + k_];    \
        static_cast<mk_trace_rec*>((p).trace)[(size_t)blockIdx.x * (p).n_phases + ph_] = r_; \
      }                                                                              \
    }                                                                                \
  } while (0)
#else
#define XR_FIELD
#define XR_INIT(s) do { } while (0)
#define XR_PUT(s, ph, slot) do { } while (0)
#define XR_MIN(s, ph, slot) do { } while (0)
#define XR_MAX(s, ph, slot) do { } while (0)
#define XR_DUMP(s, p) do { } while (0)
#endif

}  // namespace mk
