/*
 * pararnn_debug.h -- entry points of the look-back stress build of libpararnn (the same source compiled
 * with -DPR_LB_STRESS=1 into libpararnn_stress.so).  That build pauses the tiles that publish look-back
 * words (the decoupled look-back that joins time chunks in every scan; pararnn-torch README, "Method":
 * each linear solve is a parallel scan along time) for pseudo-random times, so that later tiles walk far
 * back; its results must equal the plain library's bit for bit.  The plain library does not export this.
 */
#ifndef PARARNN_DEBUG_H
#define PARARNN_DEBUG_H

#ifdef __cplusplus
extern "C" {
#endif

/* The deepest look-back walk since the last reset, counted in aggregate words passed before an
 * inclusive word was found (0: every tile found its predecessor's state at once).  Waits for the
 * device; reset != 0 clears the counter after reading it.  Returns the depth (>= 0) or
 * PARARNN_ERR_HIP (-4) when a HIP call fails. */
int pararnn_debug_lookback_depth(int reset);

#ifdef __cplusplus
}
#endif
#endif /* PARARNN_DEBUG_H */
