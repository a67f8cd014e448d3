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
 * - All entry points except qjl_release_cache are thread-safe.  Inputs with
 *   Inf or NaN give undefined (but memory-safe) results.
 * - The library is silent unless the environment (read once per process)
 *   says otherwise: QJL_LOG=1 prints every error to stderr ("[qjl] error
 *   <status>: <message>"), QJL_LOG=2 also names every call; QJL_TRACE=1 wraps
 *   every call in a roctx range (the ROCm tracer's marker API, loaded on
 *   first use), visible under rocprofv3 --marker-trace.
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

/* ---- Rotate-then-quantize tables (pure host code, no GPU needed) ----
 * "The Geometry of Forgetting", sections "Random rotation, and what high
 * dimensions do to your intuitions", "TurboQuant: bridging MSE and inner
 * product, in two stages" and "PolarQuant: skipping Cartesian altogether".
 *
 * qjl_rotation_host: the seeded random rotation Pi, fp32 [d][d] row-major
 * (y = Pi k): the Q factor of a QR of the d x d standard normals drawn from
 * `seed` exactly as S is (element e = j*d + i), with R's diagonal made
 * positive (the uniform, Haar-distributed rotation), rounded to fp32.
 * Errors: QJL_EINVAL (out NULL, d outside [2, 1024]). */
QJL_API qjl_status qjl_rotation_host(uint64_t seed, int32_t d, float *out);

/* qjl_tq_codebook_host: the 2^k centroids (ascending) of the optimal scalar
 * quantizer (Lloyd-Max) for one coordinate of a randomly rotated unit
 * vector in d dimensions, each rounded to the nearest multiple of 2^-20.
 * Cell boundaries are the midpoints of adjacent centroids.
 * Errors: QJL_EINVAL (NULL, d outside [4, 65536], k outside [1, 4]). */
QJL_API qjl_status qjl_tq_codebook_host(int32_t d, int32_t k, float *centroids);

/* qjl_pq_codebook_host: PolarQuant's codebook of one level.  Level 1
 * (angles uniform on [0, 2 pi)): 2^bits equal cells, centroids at the cell
 * middles, and the 2^bits / 4 - 1 thresholds tan(t 2 pi / 2^bits),
 * t = 1 .. 2^bits / 4 - 1, that split one quadrant.  Level l >= 2 (density
 * proportional to sin^(2^(l-1) - 1)(2 psi) on [0, pi/2]): the Lloyd-Max
 * centroids rounded to multiples of 2^-20 and the 2^bits - 1 thresholds
 * tan(midpoint of adjacent centroids).  Thresholds are rounded to multiples
 * of 2^-20.  Errors: QJL_EINVAL (NULL, level outside [1, 10], bits outside
 * [1, 5], or bits < 2 at level 1). */
QJL_API qjl_status qjl_pq_codebook_host(int32_t level, int32_t bits, float *centroids,
                                        float *thresholds);

/* TurboQuant_prod encode ("The Geometry of Forgetting", section "TurboQuant:
 * bridging MSE and inner product, in two stages"): k bits per coordinate of
 * the rotated, normalized key from the Lloyd-Max codebook
 * (qjl_tq_codebook_host(d, k)), then one QJL bit per coordinate on the
 * residual.  For each key, exactly (every decision is unique):
 *   norms  = fp32(sqrt(fp64 sum of k_j^2, channel order));
 *   y_i    = fp32 rounding (nearest even) of the exact sum_j Pi[i][j] k_j,
 *            Pi = qjl_rotation_host(seed, d);
 *   u_i    = fp32(y_i / norm) (0 for a zero key);  idx_i = number of cell
 *            boundaries (midpoints of adjacent centroids) <= u_i;
 *   r_i    = fp32(u_i - c[idx_i]);  gammas = fp32(sqrt(fp64 sum r_i^2));
 *   bit_l  = [exact sum_i S[i][l] r_i >= 0], S = the QJL sketch of seed + 1
 *            with m = d (bf16, as qjl_sketch_host(seed + 1, d, d)).
 * Layouts (rows [pos, pos + n) of every (b, h) written, others untouched):
 *   codes  uint32 [B][H_kv][cap][d k / 32]: idx_i in bits k i .. k i + k - 1
 *          of the row's bit stream (least significant bit first);
 *   bits   uint32 [B][H_kv][cap][d / 32] (as QJL sign words);
 *   norms, gammas fp32 [B][H_kv][cap].
 * keys_bf16 [B][H_kv][n][d], 16-byte aligned; d == 128; k in {1, 2, 3};
 * the other pointers 4-byte aligned.  Other sizes as for qjl_encode_keys.  The first call for a seed
 * on a device uploads its tables (~100 KB).  Returns QJL_OK, QJL_EINVAL,
 * QJL_EUNSUPPORTED, QJL_ENOMEM or QJL_EHIP. */
QJL_API qjl_status qjl_tq_encode_keys(const void *keys_bf16, int32_t B, int32_t H_kv, int32_t n,
                                      int32_t d, int32_t k, uint64_t seed, uint32_t *codes,
                                      uint32_t *bits, float *norms, float *gammas, int32_t cap,
                                      int32_t pos, void *stream);

/* Workspace bytes of qjl_tq_scores: the prepared queries of the B * H_q
 * heads, 4096 bytes each (k = 3: Pi q and S^T Pi q in fp32; k = 1, 2: their
 * integer byte-limb operands and scale factors).  0 for invalid sizes.  Pure
 * host code. */
QJL_API size_t qjl_tq_scores_workspace_bytes(int32_t B, int32_t H_q, int32_t d);

/* TurboQuant_prod scores: the estimate of <q, k_t> for every query head and
 * cached token t < N (same section: the reconstruction's inner product plus
 * the QJL estimate of the residual's, unbiased):
 *   scores[b][h][t] = norm_t (<Pi q, c[idx_t]> + sqrt(pi/2)/d gamma_t
 *                     <S^T Pi q, 2 bit_t - 1>),  kv head h / (H_q / H_kv).
 * q fp32 [B][H_q][d]; caches as written by qjl_tq_encode_keys (same k,
 * seed), codes and bits 16-byte aligned, the rest 4-byte aligned; scores
 * fp32 [B][H_q][N].  G = H_q / H_kv in {1, 2, 4, 8}; 1 <= N <= cap;
 * B, H_kv <= 65535.  workspace: device, 256-byte aligned, at least
 * qjl_tq_scores_workspace_bytes(B, H_q, d) bytes; its contents are
 * overwritten (no zero-fill needed, and a workspace shared with
 * qjl_decode_attention must be zero-filled again before that call).  fp32
 * arithmetic for k = 3; for k = 1, 2 exact integer dot products of the
 * codes' bit-planes with the query side quantized to 2^-28 of its largest
 * value, combined in fp32 (relative error ~1e-6 of the score scale).  Returns QJL_OK,
 * QJL_EINVAL, QJL_EWORKSPACE, QJL_EUNSUPPORTED, QJL_ENOMEM or QJL_EHIP. */
QJL_API qjl_status qjl_tq_scores(const float *q, const uint32_t *codes, const uint32_t *bits,
                                 const float *norms, const float *gammas, int32_t B, int32_t H_q,
                                 int32_t H_kv, int32_t N, int32_t cap, int32_t d, int32_t k,
                                 uint64_t seed, float *scores, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* PolarQuant encode ("The Geometry of Forgetting", section "PolarQuant:
 * skipping Cartesian altogether"): the rotated key y (as for
 * qjl_tq_encode_keys) is turned into polar form recursively and each angle
 * stored as its cell in the level's codebook (qjl_pq_codebook_host; 4 bits
 * at level 1, 2 bits at levels 2..7 for d = 128), with the radius in fp32:
 *   level 1, pair (a, b) = (y_2j, y_2j+1): quadrant q from the signs (the
 *     angle lies in [q pi/2, (q+1) pi/2); (0, 0) has angle 0), the pair turned
 *     into the first quadrant ((a,b), (b,-a), (-a,-b), (-b,a)) = (a', b'), cell
 *     = 4 q + #{thresholds T : b' >= T a'} (fp64; 0 for (0, 0));
 *   level l >= 2: with fp64 slice sums of squares (pairs a^2 + b^2, then sums
 *     of adjacent slices), cell = #{thresholds T : s_b >= (T T) s_a};
 *   radius = fp32(sqrt(fp64 total)).
 *   codes  uint32 [B][H_kv][cap][12]: the 64 level-1 cells (4 bits each, pair
 *          0 first), then the 63 cells of levels 2..7 (2 bits each, level
 *          by level), least significant bit first; 2 bits of padding.
 *   radii  fp32 [B][H_kv][cap].
 * d == 128; other sizes and errors as for qjl_tq_encode_keys. */
QJL_API qjl_status qjl_pq_encode_keys(const void *keys_bf16, int32_t B, int32_t H_kv, int32_t n,
                                      int32_t d, uint64_t seed, uint32_t *codes, float *radii,
                                      int32_t cap, int32_t pos, void *stream);

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
 *                (one uint32 per (batch, kv head), up to 256 bytes apart
 *                when there are few of them) that every call returns to
 *                zero; the rest is scratch that each call overwrites.  A
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

/* One decode step that first appends a token, in a single launch: token
 * `pos` of every (batch, kv head) is encoded from new_keys_bf16 (sign bits
 * of S^T k and ||k||, exactly as qjl_encode_keys defines them) into row `pos`
 * of signs / norms, its value row is copied from new_values_bf16 into row
 * `pos` of values_bf16, and query head h then attends over tokens [0, pos]
 * as in qjl_decode_attention with N = pos + 1.  (The encode: "QJL: 1-Bit
 * Quantized JL Transform ...", Abstract; "The Geometry of Forgetting", QJL
 * section; every generated token leaves a key and a value in the cache and
 * the next token attends over all of them, "The Geometry of Forgetting",
 * opening section.)
 *
 *   q                fp32 [B][H_q][d], 16-byte aligned.
 *   new_keys_bf16    bf16 [B][H_kv][d], 16-byte aligned (not inside the caches).
 *   new_values_bf16  bf16 [B][H_kv][d], 16-byte aligned (not inside the caches).
 *   signs, norms, values_bf16  the caches, [B][H_kv][cap][.], as for
 *                    qjl_decode_attention; row `pos` is written, rows
 *                    [0, pos) are read, other rows are untouched.
 *   0 <= pos < cap.  scale, out: as for qjl_decode_attention.
 *   workspace        as for qjl_decode_attention, at least
 *                    qjl_decode_workspace_bytes(B, H_q, H_kv, pos + 1, d, m).
 * The new sign words equal those qjl_encode_keys writes; the norm may differ
 * from the tile encode's in the last fp32 bit (it is the fp32 rounding of the
 * fp64 norm).  Returns QJL_OK, QJL_EINVAL, QJL_EUNSUPPORTED, QJL_EWORKSPACE,
 * QJL_ENOMEM or QJL_EHIP. */
QJL_API qjl_status qjl_decode_step(const float *q, const void *new_keys_bf16,
                                   const void *new_values_bf16, uint32_t *signs, float *norms,
                                   void *values_bf16, int32_t B, int32_t H_q, int32_t H_kv,
                                   int32_t pos, int32_t cap, int32_t d, int32_t m, uint64_t seed,
                                   float scale, float *out, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* The uncompressed baseline on the same kernel skeleton: exact scaled
 * dot-product attention over bf16 keys and values, so that the decode's
 * speed-up from 1-bit keys can be measured at equal context (the QJL page
 * claims a faster runtime than full-precision keys: "QJL: 1-Bit Quantized
 * JL Transform ...", Abstract).  Not part of the QJL method.
 *   out[b][h] = sum_t softmax_t(scale * q[b][h] . k_t) v_t over t in [0, N)
 * of kv head h / (H_q / H_kv).  q is split into three bf16 parts (their sum
 * is fp32 q to 2^-24), the products run on the bf16 matrix cores with fp32
 * accumulation; softmax, the weighted sum and the split merge are those of
 * qjl_decode_attention (same plan and workspace size:
 * qjl_decode_workspace_bytes(B, H_q, H_kv, N, d, 256)).
 *   q           fp32 [B][H_q][d], 16-byte aligned.
 *   keys_bf16   bf16 [B][H_kv][cap][d], values_bf16 likewise; 16-byte aligned.
 *   d == 128; G = H_q / H_kv in {1, 2, 4, 8}; 1 <= N <= cap; scale as for
 *   qjl_decode_attention; out fp32 [B][H_q][d]; workspace as for it.
 * Returns QJL_OK, QJL_EINVAL, QJL_EUNSUPPORTED, QJL_EWORKSPACE or QJL_EHIP. */
QJL_API qjl_status qjl_baseline_decode_attention_bf16(const float *q, const void *keys_bf16,
                                                      const void *values_bf16, int32_t B, int32_t H_q,
                                                      int32_t H_kv, int32_t N, int32_t cap, int32_t d,
                                                      float scale, float *out, void *workspace,
                                                      size_t workspace_bytes, void *stream);

/* Bytes of device scratch the library holds per GPU for
 * qjl_decode_attention_noalloc: the 4096-byte counter region plus 4 MiB of
 * split partials. */
#define QJL_NOALLOC_SCRATCH_BYTES (4096u + (4u << 20))

/* qjl_decode_attention without a workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, semantics and results as
 * qjl_decode_attention (same kernels and split plan), except:
 *   - The split scratch (arrival counters and partials) is a static array of
 *     QJL_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 *     on until the process ends.  Sizes whose plan needs more
 *     (qjl_decode_workspace_bytes(...) > QJL_NOALLOC_SCRATCH_BYTES with more
 *     than one split; only very many kv heads with G = 8 get there) return
 *     QJL_EWORKSPACE before anything is launched.
 *   - Nothing is allocated: no hipMalloc, hipFree or allocating library call.
 *     S for (seed, d, m) must already be resident on the current device
 *     (any earlier qjl_encode_keys or qjl_decode_attention call with this
 *     seed, d and m on it uploads it); otherwise QJL_EINVAL.
 *   - The first call on a device looks up the array's device address and
 *     queues a small kernel on `stream` that clears its counter region.
 *   - All calls on one GPU share its array, which keeps the last call's
 *     contents: calls that may overlap on one GPU (several streams, several
 *     threads) race and give wrong results.  Serialize them.
 * Returns QJL_OK, QJL_EINVAL, QJL_EUNSUPPORTED, QJL_EWORKSPACE or QJL_EHIP. */
QJL_API qjl_status qjl_decode_attention_noalloc(const float *q, const uint32_t *signs,
                                                const float *norms, const void *values_bf16,
                                                int32_t B, int32_t H_q, int32_t H_kv, int32_t N,
                                                int32_t cap, int32_t d, int32_t m, uint64_t seed,
                                                float scale, float *out, void *stream);

/* Frees the library's device copies of S and of the rotate-then-quantize
 * tables on every device (waiting for each device first).  Later calls
 * re-create them on demand.  Call it only while no other thread is inside a
 * qjl_* call: a call in progress may already hold the tables' addresses. */
QJL_API qjl_status qjl_release_cache(void);

#ifdef __cplusplus
}
#endif

#endif /* QJL_H */
