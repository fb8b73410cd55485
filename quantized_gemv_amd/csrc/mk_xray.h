// X-ray: per-workgroup, per-phase timestamps inside the decode kernel.
//
// The monolith page ("Design decisions", Timing; milestone M2) has lane 0 of
// warp 0 in every block write start/end stamps per phase to a preallocated
// buffer behind a compile-time flag, with the SM id, and aligns the clocks
// offline.  Here thread 0 of each workgroup records s_memtime (shader clock
// counter) at phase start, wait begin, wait end and phase end, s_memrealtime
// (100 MHz, shared by all XCDs, used for alignment) at start and end, and the
// HW_ID and XCC_ID registers.  Without MK_XRAY every macro is empty.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk.h"

namespace mk {

struct XrayClock {
#ifdef MK_XRAY
  uint64_t t_start, t_wb, t_we, rt_start;
  uint64_t mark[4];
  uint32_t active;
#endif
};

#ifdef MK_XRAY
#define XR_BEGIN(xc)                                              \
  do {                                                            \
    if (threadIdx.x == 0) {                                       \
      (xc).t_start = __builtin_amdgcn_s_memtime();                \
      (xc).rt_start = __builtin_amdgcn_s_memrealtime();           \
      (xc).t_wb = (xc).t_we = (xc).t_start;                       \
      (xc).mark[0] = (xc).mark[1] = (xc).mark[2] = (xc).mark[3] = 0; \
      (xc).active = 0;                                            \
    }                                                             \
  } while (0)
#define XR_WAIT_BEGIN(xc) do { if (threadIdx.x == 0) (xc).t_wb = __builtin_amdgcn_s_memtime(); } while (0)
#define XR_WAIT_END(xc) do { if (threadIdx.x == 0) (xc).t_we = __builtin_amdgcn_s_memtime(); } while (0)
#define XR_ACTIVE(xc) do { if (threadIdx.x == 0) (xc).active = 1; } while (0)
#define XR_MARK(xc, k) do { if (threadIdx.x == 0) (xc).mark[k] = __builtin_amdgcn_s_memtime(); } while (0)
#define XR_END(xc, p, ph_id)                                                          \
  do {                                                                                \
    if (threadIdx.x == 0 && (p).trace) {                                              \
      mk_trace_rec r;                                                                 \
      r.phase = (ph_id);                                                              \
      r.wg = blockIdx.x;                                                              \
      r.hw_id = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);                 \
      r.xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);                   \
      r.active = (xc).active;                                                         \
      r.pad = 0;                                                                      \
      r.t_start = (xc).t_start;                                                       \
      r.t_wait_begin = (xc).t_wb;                                                     \
      r.t_wait_end = (xc).t_we;                                                       \
      r.t_end = __builtin_amdgcn_s_memtime();                                         \
      r.rt_start = (xc).rt_start;                                                     \
      r.rt_end = __builtin_amdgcn_s_memrealtime();                                    \
      for (int k_ = 0; k_ < 4; ++k_) r.t_mark[k_] = (xc).mark[k_];                     \
      static_cast<mk_trace_rec*>((p).trace)[(size_t)blockIdx.x * (p).n_phases + (ph_id)] = r; \
    }                                                                                 \
  } while (0)
#else
#define XR_BEGIN(xc) do { } while (0)
#define XR_WAIT_BEGIN(xc) do { } while (0)
#define XR_WAIT_END(xc) do { } while (0)
#define XR_ACTIVE(xc) do { } while (0)
#define XR_MARK(xc, k) do { } while (0)
#define XR_END(xc, p, phase) do { } while (0)
#endif

}  // namespace mk
