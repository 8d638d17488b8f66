/* Checked build of the routed-experts library: libmoe_routed_checked.so.
 *
 * The same sources as libmoe_routed.so compiled with MOE_CHECKED. It exports every entry point of
 * moe_routed.h with the same behaviour, and in addition its kernels test each global memory access
 * against the extent of the buffer it belongs to (the plan's arrays, the routed and token rows,
 * the weights, the outputs, the weight gradients; the router kernels are not instrumented). An
 * access outside its buffer is not made: a copy or store is skipped and a load reads zeros, so a
 * wrong index yields wrong values and a count instead of a memory fault. The tests below run
 * slower than the product build (their bookkeeping spills registers in the GEMMs).
 *
 * For: the library's own tests and the debugging of shapes or call sequences suspected of
 * touching memory outside their buffers. Not for production use; libmoe_routed.so does not
 * export these functions.
 */
#ifndef MOE_ROUTED_CHECKED_H
#define MOE_ROUTED_CHECKED_H

#include <stdint.h>

#include "moe_routed.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of accesses found outside their buffer since the library was loaded or last reset,
 * summed over all kernels. Waits for the whole device first (hipDeviceSynchronize).
 * count: host pointer, written on success. Returns MOE_OK, MOE_E_NULL (count is NULL) or
 * MOE_E_HIP. */
moe_status moe_checked_violations(uint64_t* count);

/* Sets the violation count to zero (after waiting for the device). Returns MOE_OK or MOE_E_HIP. */
moe_status moe_checked_reset(void);

/* Test of the checks themselves: every buffer extent the grouped GEMMs test against is taken as
 * `bytes` shorter than it is, so that valid accesses near the end of a buffer are counted as
 * violations (and skipped) while no access leaves its real buffer. 0 (the default) restores the
 * true extents. Host state of this process; affects launches made after the call. Returns MOE_OK,
 * or MOE_E_SHAPE for bytes < 0. */
moe_status moe_checked_shrink(int64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTED_CHECKED_H */
