/*
 * qjl_testing.h - test hooks of libqjl.so.  Not part of the public C ABI
 * (include/qjl.h); the library's own tests use them to run either encode
 * kernel on any key count.
 */
#ifndef QJL_TESTING_H
#define QJL_TESTING_H

#include <stdint.h>

#include "qjl.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Encode calls made by the CALLING THREAD with at most `keys` keys
 * (B * H_kv * n) run the small-set kernel (fp64 projections, four lanes per
 * key and sketch coordinate); larger ones run the tile kernel.  The default
 * is 512.  Calls above 2^21 keys (2^20 at m = 512) always run the tile
 * kernel; 0 sends every call to the tile kernel; a negative `keys` changes
 * nothing.  Returns the thread's previous limit.  Other threads keep their
 * own limit, so the hook never changes another thread's routing.  Both
 * kernels give identical sign words; norms may differ in the last bit. */
QJL_API int32_t qjl_testing_set_encode_small_max(int32_t keys);

/* Rotate-then-quantize encodes (qjl_tq_encode_keys, qjl_pq_encode_keys)
 * made by the CALLING THREAD widen their two error certificates (the fp32
 * rounding of the rotated key, the signs of the residual's sketch) by
 * 2^log2_factor, so that many values take the exact integer paths; the
 * results must not change.  0 (the default) is the production margin;
 * values outside [0, 60] change nothing.  Returns the previous value. */
QJL_API int32_t qjl_testing_set_rotq_margin(int32_t log2_factor);

#ifdef __cplusplus
}
#endif

#endif /* QJL_TESTING_H */
