// Host-side helpers of libgtattn: status plumbing, the per-thread error
// detail, and the optional per-kernel event timing.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gt_attn.h"
#include "../../include/gt_proj.h"

namespace gt {

// Record a failure detail for gt_last_error() and return the status.
gt_status fail(gt_status s, const char *fmt, ...);
void clear_error();

// hipError_t -> GT_E_HIP with the runtime's message.
#define GT_HIP(expr)                                                        \
  do {                                                                      \
    hipError_t e_ = (expr);                                                 \
    if (e_ != hipSuccess)                                                   \
      return ::gt::fail(GT_E_HIP, "%s: %s", #expr, hipGetErrorString(e_));  \
  } while (0)

#define GT_CHECK_LAUNCH()                                                   \
  do {                                                                      \
    hipError_t e_ = hipGetLastError();                                      \
    if (e_ != hipSuccess)                                                   \
      return ::gt::fail(GT_E_HIP, "launch at %s:%d: %s", __FILE__, __LINE__, \
                        hipGetErrorString(e_));                             \
  } while (0)

// Per-kernel event timing (gt_prof_enable).  prof_begin returns a token
// that prof_end closes after the launch.
enum ProfKernel { PK_FWD = 0, PK_FWD_MERGE, PK_BWD_ROWS, PK_BWD_ROWS_MERGE, PK_BWD_COLS,
                  PK_BWD_COLS_MERGE, PK_BWD_DBIAS, PK_COUNT };
int prof_begin(ProfKernel k, hipStream_t s);
void prof_end(int token, hipStream_t s);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace gt
