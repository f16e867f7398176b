/*
 * pararnn_debug.h -- entry points of the look-back stress build of libpararnn (the same source compiled
 * with -DPR_LB_STRESS=1 into libpararnn_stress.so).  That build pauses the tiles that publish look-back
 * words (the decoupled look-back that joins time chunks in every scan; pararnn-torch README, "Method":
 * the linearised system is solved by a parallel scan along time) for pseudo-random times, so that tiles
 * take their carry by either path; its results must equal the plain library's bit for bit.  The plain
 * library does not export this.
 */
#ifndef PARARNN_DEBUG_H
#define PARARNN_DEBUG_H

#ifdef __cplusplus
extern "C" {
#endif

/* The deepest look-back walk since the last reset: the most aggregates any tile passed before it met an
 * inclusive word.  0 when every tile took its carry from its predecessor's inclusive word; 1 once some tile
 * took it from its predecessor's aggregate applied to the inclusive word before that (the deepest the
 * scalar and 2x2 kernels and every VJP go); the sLSTM Newton iteration walks on past as many aggregates as
 * are out.  Waits for the device; reset != 0 clears the counter after reading it.  Returns the depth (>= 0)
 * or PARARNN_ERR_HIP (-4) when a HIP call fails. */
int pararnn_debug_lookback_depth(int reset);

#ifdef __cplusplus
}
#endif
#endif /* PARARNN_DEBUG_H */
