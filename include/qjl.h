/*
 * qjl.h - C ABI of the QJL KV-cache library for AMD Instinct MI355X (gfx950).
 *
 * QJL compresses attention keys to the signs of a Johnson-Lindenstrauss
 * sketch: a key k is replaced by the m bits sign(S^T k) plus its norm ||k||,
 * with no per-block zero point or scale ("QJL: 1-Bit Quantized JL Transform
 * for KV Cache Quantization with Zero Overhead", Abstract).  A decode step
 * estimates every <q, k> from those bits with the asymmetric estimator
 * sqrt(pi/2)/m * ||k|| * <S^T q, sign(S^T k)> (unbiased; "The Geometry of
 * Forgetting: How Three Papers Cracked KV Cache Quantization", section "QJL:
 * one bit, zero parameters, unbiased inner products"), takes the softmax of
 * the scaled estimates and the weighted sum of the bf16 values.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - S is a d x m matrix with i.i.d. standard normal entries drawn from a
 *   64-bit seed (same section: S is regenerated from a seed, never stored by
 *   the caller).  Element e = j*m + i (row j = key channel, column i = sketch
 *   coordinate) is member (e mod 2) of the Box-Muller pair e / 2, built from
 *   SplitMix64 outputs 2*(e/2)+1 and 2*(e/2)+2 of the stream started at
 *   `seed`; each output r is mapped to ((r >> 11) + 1) * 2^-53 in (0, 1].
 *   The normal is rounded to fp32 and then to bf16 (nearest, ties to even);
 *   both encode and decode use these bf16 values.
 * - Bit i of a key is 1 iff the exact real sum over j of k_j * S[j][i] is
 *   >= 0 (a zero sum gives +1).  The library certifies every bit: matrix-core
 *   sums too close to zero to trust are re-evaluated exactly on the GPU.
 * - Bits are packed 32 per uint32 word, coordinate 32*w + b in bit b of word
 *   w (least significant bit first), m/32 words per key.
 * - Supported shapes: d == 128; m == 256 or m == 512; for decode,
 *   H_q % H_kv == 0 with G = H_q / H_kv in {1, 2, 4, 8}.  Other values return
 *   QJL_EUNSUPPORTED.
 * - Device pointers are HIP device memory of the current device.  `stream`
 *   is a hipStream_t (NULL = the default stream).  Calls enqueue their
 *   kernel launches (one, or a few for large encode calls) on `stream` and
 *   return without waiting; errors inside a kernel surface at
 *   the caller's next synchronization.  The first call for a given
 *   (device, seed, d, m) uploads S to the device synchronously and keeps it
 *   until qjl_release_cache() or process exit.
 * - Validation runs before any HIP call: on an error return nothing has been
 *   launched and no output has been written.
 * - All entry points are thread-safe.  Inputs with Inf or NaN give undefined
 *   (but memory-safe) results.
 */
#ifndef QJL_H
#define QJL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define QJL_API __attribute__((visibility("default")))
#else
#define QJL_API
#endif

typedef int32_t qjl_status;

enum {
  QJL_OK = 0,
  QJL_EINVAL = 1,         /* null or misaligned pointer, bad size or range   */
  QJL_EUNSUPPORTED = 2,   /* d, m or G outside the supported set             */
  QJL_EWORKSPACE = 3,     /* workspace pointer null/misaligned or too small  */
  QJL_EHIP = 4,           /* a HIP runtime call failed; see qjl_last_error() */
  QJL_ENOMEM = 5          /* device allocation for the S cache failed        */
};

/* Layout/semantics version of the packed bits and norms (bumped on change). */
QJL_API int32_t qjl_abi_version(void);

/* Text of the last error on the calling thread ("" if none).  The pointer
 * stays valid until the next qjl_* call on this thread. */
QJL_API const char *qjl_last_error(void);

/* The bf16 bit patterns of S for (seed, d, m), row-major [d][m], written to
 * the caller's host buffer `out` (d*m uint16).  Pure host code, no GPU needed.
 * The matrix is the one defined above (page "The Geometry of Forgetting",
 * QJL section: Gaussian S regenerated from a seed).
 * Errors: QJL_EINVAL (out == NULL, d <= 0, m <= 0, d*m > 2^26). */
QJL_API qjl_status qjl_sketch_host(uint64_t seed, int32_t d, int32_t m, uint16_t *out);

/* Encode n new keys per (batch, kv head): sign bits of S^T k plus ||k||.
 * ("QJL: 1-Bit Quantized JL Transform ...", Abstract: JL transform then sign
 *  bits, no quantization constants; "The Geometry of Forgetting", QJL
 *  section: Q(x) = sign(Sx).)
 *
 *   keys_bf16  device, bf16 [B][H_kv][n][d], contiguous, 16-byte aligned.
 *   signs      device, uint32 [B][H_kv][cap][m/32], 16-byte aligned; rows
 *              [pos, pos+n) of every (b, h) are written, others untouched.
 *   norms      device, fp32 [B][H_kv][cap], 4-byte aligned; same rows.
 *              norms = the Euclidean norm of the bf16 key in fp32 (an fp32
 *              sum of squares and the hardware square root: a few ulps).
 *   B, H_kv >= 1; n >= 0 (n == 0 is a no-op); cap >= 1; 0 <= pos;
 *   pos + n <= cap; B * H_kv * n <= 2^31 - 1 (QJL_EINVAL beyond: the
 *   kernel indexes keys in 32 bits); d == 128; m in {256, 512}.
 * The work is enqueued on `stream` and the call returns.  On a 256-CU
 * device one kernel launch takes up to 9 * 2^17 keys at m = 256 (9 * 2^16 at
 * m = 512); larger key sets are divided evenly among the fewest launches.
 * The caller owns all buffers.  Returns QJL_OK, QJL_EINVAL, QJL_EUNSUPPORTED,
 * QJL_ENOMEM (first use of this S on this device) or QJL_EHIP. */
QJL_API qjl_status qjl_encode_keys(const void *keys_bf16, int32_t B, int32_t H_kv, int32_t n,
                                   int32_t d, int32_t m, uint64_t seed, uint32_t *signs,
                                   float *norms, int32_t cap, int32_t pos, void *stream);

/* Encode calls with at most `keys` keys (B * H_kv * n) run a small-set kernel
 * (four lanes per key and sketch coordinate, fp64 projections with the same
 * exact-sign guarantee); larger calls run the tile kernel.  The default, 512,
 * covers a decode step that appends one token per (batch, kv head) for up to
 * 512 such pairs; alone, the two kernels take equal time near 800 keys at
 * m = 256 and 550 at m = 512.  Calls above 2^21 keys (2^20 at m = 512) always run the
 * tile kernel.  0 sends
 * every call to the tile kernel.  A negative `keys` changes nothing.  Returns
 * the previous limit.  Process-wide; takes effect for calls made after it
 * returns.  (For tuning and for testing either kernel on any size.) */
QJL_API int32_t qjl_set_encode_small_max(int32_t keys);

/* Number of context splits a decode call with these sizes uses (>= 1); 0 on
 * invalid sizes.  Pure host code. */
QJL_API int32_t qjl_decode_num_splits(int32_t B, int32_t H_q, int32_t H_kv, int32_t N,
                                      int32_t d, int32_t m);

/* Workspace bytes qjl_decode_attention needs for these sizes; 0 on invalid
 * sizes.  Pure host code.  The workspace holds per-split partial softmax
 * states and one arrival counter per (batch, kv head). */
QJL_API size_t qjl_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv, int32_t N,
                                          int32_t d, int32_t m);

/* One decode step of QJL attention.  Query head h of batch b attends over
 * cached tokens [0, N) of kv head h / (H_q / H_kv):
 *   est_t = sqrt(pi/2)/m * norms[t] * sum_i (S^T q)_i * (2*bit_t,i - 1)
 *   out   = sum_t softmax_t(scale * est) * values[t]
 * (asymmetric estimator: "QJL: 1-Bit Quantized JL Transform ...", Abstract;
 *  constant and unbiasedness: "The Geometry of Forgetting", QJL section;
 *  "attention scores are inner products", same section.)
 *
 *   q            device fp32 [B][H_q][d], 16-byte aligned.
 *   signs, norms as written by qjl_encode_keys (same m, seed), [.][.][cap].
 *   values_bf16  device bf16 [B][H_kv][cap][d], 16-byte aligned.
 *   1 <= N <= cap.  scale > 0, or scale == 0 for 1/sqrt(d).
 *   out          device fp32 [B][H_q][d], 16-byte aligned, written whole.
 *   workspace    device, 256-byte aligned, at least
 *                qjl_decode_workspace_bytes(...) bytes, zero-filled before
 *                its first use.  Its first 4096 bytes hold arrival counters
 *                (one uint32 per (batch, kv head)) that every call returns
 *                to zero; the rest is scratch that each call overwrites.  A
 *                workspace can therefore be reused by later calls of any
 *                size on the same stream; calls that may overlap (other
 *                streams) must not share one.
 * Returns QJL_OK, QJL_EINVAL, QJL_EUNSUPPORTED, QJL_EWORKSPACE, QJL_ENOMEM or
 * QJL_EHIP. */
QJL_API qjl_status qjl_decode_attention(const float *q, const uint32_t *signs, const float *norms,
                                        const void *values_bf16, int32_t B, int32_t H_q,
                                        int32_t H_kv, int32_t N, int32_t cap, int32_t d,
                                        int32_t m, uint64_t seed, float scale, float *out,
                                        void *workspace, size_t workspace_bytes, void *stream);

/* Frees the library's device copies of S on every device (waits for the
 * device first).  Later calls re-create them on demand. */
QJL_API qjl_status qjl_release_cache(void);

#ifdef __cplusplus
}
#endif

#endif /* QJL_H */
