/*
 * moe_timing.h -- optional per-kernel timing for benchmarks (not needed to run
 * the layer).  When a launch site is armed, each launch the library makes at
 * that site records a hipEvent pair around the kernel on the kernel's own
 * stream, so a benchmark can time one kernel inside moe_forward without
 * changing the launch sequence.  Unarmed sites cost one relaxed atomic load.
 *
 * This is the only state the library keeps between calls, and only while a
 * site is armed: the events are created by moe_timing_arm and destroyed by
 * moe_timing_read.  Arm/read are host calls; they are not meant to overlap a
 * concurrent call on another thread that launches at the same site.
 */
#ifndef MOE_TIMING_H
#define MOE_TIMING_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_site {
  MOE_SITE_ROUTER_LOGITS = 0,   /* router GEMM (partial logits) */
  MOE_SITE_ROUTER_TOPK = 1,     /* top-k selection and gates */
  MOE_SITE_SORT = 2,            /* stable counting sort (3 kernels, timed together) */
  MOE_SITE_GATHER = 3,          /* row gather (+ fp8 quantisation) */
  MOE_SITE_GATE_UP = 4,         /* grouped gate/up GEMM + SwiGLU: the routed experts, and inside
                                   moe_forward also the shared expert's tiles (one launch) */
  MOE_SITE_DOWN = 5,            /* grouped down GEMM (same groups as MOE_SITE_GATE_UP) */
  MOE_SITE_SHARED_GATE_UP = 6,  /* reserved (no launch records here at present) */
  MOE_SITE_SHARED_DOWN = 7,     /* reserved (no launch records here at present) */
  MOE_SITE_COMBINE = 8,         /* weighted combine */
  MOE_SITE_BWD_DGRAD = 9,       /* backward: row-grouped GEMMs (z recompute, dy W_down, dz W_gate_up) */
  MOE_SITE_BWD_WGRAD = 10,      /* backward: token-grouped weight-gradient GEMMs */
  MOE_SITE_COUNT = 11
} moe_site;

/* Arm `site` for its next `capacity` launches (capacity in [1, 100000]).
 * MOE_EINVAL for an unknown site or capacity; MOE_EHIP if event creation fails. */
moe_status moe_timing_arm(int32_t site, int32_t capacity);

/* Wait for the site's recorded events, return the summed kernel time in
 * milliseconds and the number of timed launches, then disarm the site and
 * free its events.  A site that was never armed reads 0 ms and 0 launches. */
moe_status moe_timing_read(int32_t site, double *total_ms, int32_t *launches);

#ifdef __cplusplus
}
#endif
#endif
